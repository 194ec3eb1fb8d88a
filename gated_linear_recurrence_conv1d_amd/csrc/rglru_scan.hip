// rglru_scan.hip -- fused conv + gate nonlinearity + RG-LRU linear scan.
//
// h_t = a_t h_{t-1} + sqrt(1 - a_t^2) (i_t xc_t) with a diagonal recurrence (Soham De's Griffin
// thread, tweet on S4D/LRU's diagonal recurrent matrix), so every channel is an independent
// first-order recurrence: one lane owns one (b, d) channel and keeps its fp32 state in a register.
// The conv output xc is recomputed from x with four taps held in registers (cheaper than storing
// it); the pre-activations come from the gate projection. Loads run one group of steps ahead of
// the arithmetic so that HBM latency overlaps the gate math of the current group.
//
// The pages note that the scan is memory-bound and that its HBM traffic is what to optimise
// (Soham De's thread, tweet on the Pallas kernel); here each element costs x (in), one (pa, px)
// pair (in) and y (out) in HBM, and nothing else.
//
// Long sequences with few channels (little parallelism across lanes) use the chunked form: the
// affine maps h -> a h + u compose associatively, (A2, U2) o (A1, U1) = (A2 A1, A2 U1 + U2), so
//   pass 1 reduces each time chunk to (sum of log a, state reached from 0),
//   pass 2 prefixes those summaries across chunks (a wavefront scan over chunk index),
//   pass 3 re-scans each chunk from its carry-in and writes y.
#include "rglru_device.h"
#include "rglru_launch.h"

namespace rglru {

constexpr int kScanThreads = 256;
constexpr int kGroup = 4;  // steps per load group (4, 8, 12, 16 measured: 4 fastest, 8 within 2-8%)

template <typename T> struct StepData {
  float x[kGroup];
  typename PrePair<T>::type p[kGroup];
};

// The loads of steps [t, min(t + kGroup, tend)); xp / pp point at step t of the channel.
template <typename T>
__device__ __forceinline__ void load_group(StepData<T> &s, const T *xp,
                                           const typename PrePair<T>::type *pp, int n, int D) {
#pragma unroll
  for (int u = 0; u < kGroup; ++u) {
    if (u < n) {
      s.x[u] = Elem<T>::load(xp, 0);
      s.p[u] = *pp;
    }
    xp += D;
    pp += D;
  }
}

// Runs steps [t, t + n) (n <= kGroup) of one channel; yp points at step t. WRITE: store y;
// otherwise only advance the state and the sum of log a. NH: some channel of the wave has
// kd < -1/4, so log a can leave the polynomial's range [-1/4, 0] (a wave-uniform choice: the
// usual decays never pay for the exp2 of the other branch).
template <typename T, bool WRITE, bool NH>
__device__ __forceinline__ void run_group(const StepData<T> &s, const float (&w)[4], float kd,
                                          float (&xm)[3], float &h, float &slog, T *yp, int n,
                                          int D) {
#pragma unroll
  for (int u = 0; u < kGroup; ++u) {
    if (u < n) {
      const float xv = s.x[u];
      const float xc = fmaf(w[3], xv, fmaf(w[2], xm[2], fmaf(w[1], xm[1], w[0] * xm[0])));
      xm[0] = xm[1];
      xm[1] = xm[2];
      xm[2] = xv;
      const float pa = PrePair<T>::pa(s.p[u]);
      const float px = PrePair<T>::px(s.p[u]);
      const float r = fast_sigmoid(pa);
      const float ig = fast_sigmoid(px);
      const float z = kd * r;
      const float e = NH ? expm1_nonpos(z) : expm1_poly(z);
      const float a = 1.0f + e;
      const float m = __builtin_amdgcn_sqrtf(-e * (2.0f + e));
      h = fmaf(a, h, m * (ig * xc));
      if (WRITE) {
        Elem<T>::store(yp, 0, h);
      } else {
        slog += z;
      }
    }
    if (WRITE) yp += D;
  }
}

// Scans steps [tbeg, tend) of channel (b, d) starting from state h. Returns the final state;
// when !WRITE also the sum of log a over the range. Pointers advance by D per step (no 64-bit
// index arithmetic per access).
template <typename T, bool WRITE, bool NH>
__device__ __forceinline__ float scan_range_nh(const T *__restrict__ xb,
                                               const typename PrePair<T>::type *__restrict__ pb,
                                               T *__restrict__ yb, const float (&w)[4], float kd,
                                               int tbeg, int tend, int D, float h, float &slog) {
  float xm[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int s = tbeg - 3 + k;
    xm[k] = (s >= 0) ? Elem<T>::load(xb, static_cast<size_t>(s) * D) : 0.0f;
  }
  slog = 0.0f;
  const size_t o = static_cast<size_t>(tbeg) * D;
  const T *xp = xb + o;
  const typename PrePair<T>::type *pp = pb + o;
  T *yp = WRITE ? yb + o : nullptr;
  const size_t stride = static_cast<size_t>(kGroup) * D;
  StepData<T> cur, nxt;
  int t = tbeg;
  if (t < tend) load_group<T>(cur, xp, pp, tend - t, D);
  while (t < tend) {
    const int tn = t + kGroup;
    xp += stride;
    pp += stride;
    if (tn < tend) load_group<T>(nxt, xp, pp, tend - tn, D);
    run_group<T, WRITE, NH>(cur, w, kd, xm, h, slog, yp, tend - t, D);
    if (WRITE) yp += stride;
    cur = nxt;
    t = tn;
  }
  return h;
}

template <typename T, bool WRITE>
__device__ __forceinline__ float scan_range(const T *__restrict__ xb,
                                            const typename PrePair<T>::type *__restrict__ pb,
                                            T *__restrict__ yb, const float (&w)[4], float kd,
                                            int tbeg, int tend, int D, float h, float &slog) {
  if (__builtin_amdgcn_readfirstlane(__any(kd < -0.25f) ? 1 : 0))
    return scan_range_nh<T, WRITE, true>(xb, pb, yb, w, kd, tbeg, tend, D, h, slog);
  return scan_range_nh<T, WRITE, false>(xb, pb, yb, w, kd, tbeg, tend, D, h, slog);
}

template <typename T>
__device__ __forceinline__ void channel_params(const T *conv_w, const float *Lambda, int d, int D,
                                               float (&w)[4], float &kd) {
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = Elem<T>::load(conv_w, static_cast<size_t>(j) * D + d);
  kd = decay_coeff(Lambda[d]);
}

// ---- direct plan -----------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kScanThreads) void scan_direct(
    const T *__restrict__ x, const typename PrePair<T>::type *__restrict__ pre,
    const T *__restrict__ conv_w, const float *__restrict__ Lambda, const float *__restrict__ h0,
    T *__restrict__ y, float *__restrict__ h_T, int B, int Tn, int D) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * kScanThreads + threadIdx.x;
  if (idx >= static_cast<size_t>(B) * D) return;
  const int b = static_cast<int>(idx / D);
  const int d = static_cast<int>(idx % D);
  float w[4], kd;
  channel_params<T>(conv_w, Lambda, d, D, w, kd);
  const size_t base = static_cast<size_t>(b) * Tn * D + d;
  float slog;
  float h = h0 ? h0[idx] : 0.0f;
  h = scan_range<T, true>(x + base, pre + base, y + base, w, kd, 0, Tn, D, h, slog);
  if (h_T) h_T[idx] = h;
}

// ---- chunked plan ----------------------------------------------------------------------------
// Pass 1: grid (lanes over B*D, chunks). sums[b][c][d] = (sum log a, state from 0).
template <typename T>
__global__ __launch_bounds__(kScanThreads) void scan_chunk_summary(
    const T *__restrict__ x, const typename PrePair<T>::type *__restrict__ pre,
    const T *__restrict__ conv_w, const float *__restrict__ Lambda, float2 *__restrict__ sums,
    int B, int Tn, int D, int L, int nC) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * kScanThreads + threadIdx.x;
  if (idx >= static_cast<size_t>(B) * D) return;
  const int c = blockIdx.y;
  const int b = static_cast<int>(idx / D);
  const int d = static_cast<int>(idx % D);
  float w[4], kd;
  channel_params<T>(conv_w, Lambda, d, D, w, kd);
  const size_t base = static_cast<size_t>(b) * Tn * D + d;
  const int tbeg = c * L;
  const int tend = min(Tn, tbeg + L);
  float slog;
  const float hloc = scan_range<T, false>(x + base, pre + base, nullptr, w, kd, tbeg, tend, D,
                                          0.0f, slog);
  sums[(static_cast<size_t>(b) * nC + c) * D + d] = make_float2(slog, hloc);
}

// Pass 2: one wave per channel (b, d); lane k holds chunk k of a window of 64 chunks. An
// inclusive Hillis-Steele scan of the affine summaries across lanes, then the exclusive carry
// into each chunk; windows are chained through the running carry.
__global__ __launch_bounds__(kScanThreads) void scan_chunk_carry(
    const float2 *__restrict__ sums, const float *__restrict__ h0, float *__restrict__ carry,
    float *__restrict__ h_T, int B, int D, int nC) {
  const int lane = threadIdx.x & 63;
  const size_t ch = static_cast<size_t>(blockIdx.x) * (kScanThreads / 64) + (threadIdx.x >> 6);
  if (ch >= static_cast<size_t>(B) * D) return;  // whole wave exits together
  const int b = static_cast<int>(ch / D);
  const int d = static_cast<int>(ch % D);
  float run = h0 ? h0[ch] : 0.0f;
  for (int c0 = 0; c0 < nC; c0 += 64) {
    const int c = c0 + lane;
    float2 s = (c < nC) ? sums[(static_cast<size_t>(b) * nC + c) * D + d] : make_float2(0.f, 0.f);
    float L = s.x, Hh = s.y;  // identity map for lanes past the end: (0, 0)
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float Lp = __shfl_up(L, off, 64);
      const float Hp = __shfl_up(Hh, off, 64);
      if (lane >= off) {
        Hh = fmaf(__expf(L), Hp, Hh);
        L += Lp;
      }
    }
    // exclusive prefix: the map composed from chunk c0 .. c-1
    float Le = __shfl_up(L, 1, 64);
    float He = __shfl_up(Hh, 1, 64);
    if (lane == 0) {
      Le = 0.0f;
      He = 0.0f;
    }
    if (c < nC) carry[(static_cast<size_t>(b) * nC + c) * D + d] = fmaf(__expf(Le), run, He);
    const float Lt = __shfl(L, 63, 64);
    const float Ht = __shfl(Hh, 63, 64);
    run = fmaf(__expf(Lt), run, Ht);
  }
  if (h_T && lane == 0) h_T[ch] = run;
}

// Pass 3: re-scan every chunk from its carry-in and write y.
template <typename T>
__global__ __launch_bounds__(kScanThreads) void scan_chunk_final(
    const T *__restrict__ x, const typename PrePair<T>::type *__restrict__ pre,
    const T *__restrict__ conv_w, const float *__restrict__ Lambda,
    const float *__restrict__ carry, T *__restrict__ y, int B, int Tn, int D, int L, int nC) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * kScanThreads + threadIdx.x;
  if (idx >= static_cast<size_t>(B) * D) return;
  const int c = blockIdx.y;
  const int b = static_cast<int>(idx / D);
  const int d = static_cast<int>(idx % D);
  float w[4], kd;
  channel_params<T>(conv_w, Lambda, d, D, w, kd);
  const size_t base = static_cast<size_t>(b) * Tn * D + d;
  const int tbeg = c * L;
  const int tend = min(Tn, tbeg + L);
  float slog;
  const float hin = carry[(static_cast<size_t>(b) * nC + c) * D + d];
  scan_range<T, true>(x + base, pre + base, y + base, w, kd, tbeg, tend, D, hin, slog);
}

// ----------------------------------------------------------------------------------------------
template <typename T>
static hipError_t direct_impl(const void *x, const void *pre, const void *conv_w,
                              const float *Lambda, const float *h0, void *y, float *h_T, int B,
                              int Tn, int D, hipStream_t s) {
  const size_t lanes = static_cast<size_t>(B) * D;
  const unsigned blocks = static_cast<unsigned>((lanes + kScanThreads - 1) / kScanThreads);
  scan_direct<T><<<blocks, kScanThreads, 0, s>>>(
      static_cast<const T *>(x), static_cast<const typename PrePair<T>::type *>(pre),
      static_cast<const T *>(conv_w), Lambda, h0, static_cast<T *>(y), h_T, B, Tn, D);
  return hipGetLastError();
}

template <typename T>
static hipError_t chunked_impl(const void *x, const void *pre, const void *conv_w,
                               const float *Lambda, const float *h0, void *y, float *h_T, int B,
                               int Tn, int D, int L, float2 *sums, float *carry, hipStream_t s) {
  const int nC = (Tn + L - 1) / L;
  const size_t lanes = static_cast<size_t>(B) * D;
  dim3 grid(static_cast<unsigned>((lanes + kScanThreads - 1) / kScanThreads), nC);
  const T *xx = static_cast<const T *>(x);
  const typename PrePair<T>::type *pp = static_cast<const typename PrePair<T>::type *>(pre);
  const T *cw = static_cast<const T *>(conv_w);
  scan_chunk_summary<T><<<grid, kScanThreads, 0, s>>>(xx, pp, cw, Lambda, sums, B, Tn, D, L, nC);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned cblocks = static_cast<unsigned>((lanes + 3) / 4);
  scan_chunk_carry<<<cblocks, kScanThreads, 0, s>>>(sums, h0, carry, h_T, B, D, nC);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  scan_chunk_final<T><<<grid, kScanThreads, 0, s>>>(xx, pp, cw, Lambda, carry,
                                                    static_cast<T *>(y), B, Tn, D, L, nC);
  return hipGetLastError();
}

hipError_t launch_scan_direct(const void *x, const void *pre, const void *conv_w,
                              const float *Lambda, const float *h0, void *y, float *h_T, int B,
                              int T, int D, int io, hipStream_t s) {
  if (io == kBF16) return direct_impl<bf16_t>(x, pre, conv_w, Lambda, h0, y, h_T, B, T, D, s);
  return direct_impl<float>(x, pre, conv_w, Lambda, h0, y, h_T, B, T, D, s);
}

hipError_t launch_scan_chunked(const void *x, const void *pre, const void *conv_w,
                               const float *Lambda, const float *h0, void *y, float *h_T, int B,
                               int T, int D, int L, float2 *sums, float *carry, int io,
                               hipStream_t s) {
  if (io == kBF16)
    return chunked_impl<bf16_t>(x, pre, conv_w, Lambda, h0, y, h_T, B, T, D, L, sums, carry, s);
  return chunked_impl<float>(x, pre, conv_w, Lambda, h0, y, h_T, B, T, D, L, sums, carry, s);
}

}  // namespace rglru
