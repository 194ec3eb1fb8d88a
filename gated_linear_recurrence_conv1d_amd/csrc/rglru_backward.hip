// rglru_backward.hip -- gradients of the Conv1D(width 4) -> RG-LRU forward.
//
// The forward (Griffin paper page on docshare.wps.com, section "Model Architecture"; the gate
// that can discard the input and keep the history, Soham De's Griffin thread, tweet on adding a
// Recurrent Gate to LRU; the temporal Conv1D in front, same thread, tweet on keeping the recurrent
// block simple) is differentiated with the chain rule. The pages name training as the place the
// method was memory bound (same thread, the tweet on the Pallas kernel and HBM accesses), which
// is why this pass exists; they print no backward. Notation, per (b, d) and time t:
//   delta_t = dL/dh_t = dy_t + g_{t+1},   g_t = a_t delta_t,   g_T = dh_T,   dh0 = g_0
// (g_t is the gradient that step t passes to h_{t-1}; it obeys the same kind of affine recurrence
// as the forward, run backward in time). With z = log a = kd r, e = expm1(z), m = sqrt(1 - a^2):
//   dm = delta i xc, di = delta m xc, da = delta h_{t-1},
//   dz = da a - dm a^2 / m          (dm/dz = -a^2/m; the term is 0 where m = 0)
//   dpa = kd dz r (1 - r),  dpx = di i (1 - i),  dxc = delta m i + (W_a^T dpa + W_x^T dpx),
//   dLambda = 8 sigmoid(-Lambda) sum_t r dz,  db = sum_t dp,  dW = sum_t dp xc^T,
//   dx[s] = sum_j conv_w[j] dxc[s + 3 - j],  dconv_w[j] = sum_t dxc[t] x[t - 3 + j].
// h_{t-1} is read from the forward's output y (the state rounded to the I/O dtype) and h0.
//
// Passes, each one kernel:
//  1. bwd_summary: per (b, d, chunk of kBwdChunk steps) the chunk's map g_start = P g_end + Q
//     (P = product of a over the chunk, Q = g_start from g_end = 0), walking the chunk backward.
//  2. bwd_carry: per (b, d) the g entering every chunk from its right, and dh0.
//  3. bwd_emit: per (b, d, chunk) the backward walk from that carry: writes (dpa, dpx) pairs,
//     the direct part of dxc, and per-chunk partial sums of dpa, dpx and r dz.
//  4. dxc_mfma / dxc_valu: dxc += [dpa dpx] [W_a ; W_x] per head (bf16 MFMA or fp32 VALU).
//  5. conv_bwd: dx from dxc and conv_w; per-chunk partials of dconv_w.
//  6. dw_mfma / dw_valu: per head and row split, partial dW = dp^T xc with xc recomputed from x.
//  7. bwd_reduce: fixed-order sums of all partials (deterministic: no floating-point atomics).
#include <algorithm>

#include "rglru_launch.h"
#include "rglru_mfma.h"

namespace rglru {

constexpr int kBwdThreads = 256;

// (dpa, dpx) pair storage. fp32 I/O: one float2 (dpa first). bf16 I/O: the pair rounded to two
// bf16 (dpa in the low half) in `hi`, and the rounding residuals, again as a bf16 pair, in `lo`:
// hi + lo carries about 16 significant bits, which the dW contraction needs (see dw_mfma); the
// dxc contraction reads hi alone.
template <typename T> struct DPair;
template <> struct DPair<float> {
  typedef float2 type;
  __device__ __forceinline__ static void put(type *hi, type *, size_t o, float a, float x) {
    hi[o] = make_float2(a, x);
  }
  __device__ __forceinline__ static void get(const type *hi, const type *, size_t o, float &a,
                                             float &x) {
    const float2 v = hi[o];
    a = v.x;
    x = v.y;
  }
};
template <> struct DPair<bf16_t> {
  typedef uint32_t type;
  __device__ __forceinline__ static void put(type *hi, type *lo, size_t o, float a, float x) {
    const uint32_t h = pack_bf16x2(a, x);
    hi[o] = h;
    lo[o] = pack_bf16x2(a - bf16lo(h), x - bf16hi(h));  // the differences are exact in fp32
  }
  __device__ __forceinline__ static void get(const type *hi, const type *lo, size_t o, float &a,
                                             float &x) {
    const uint32_t h = hi[o], l = lo[o];
    a = bf16lo(h) + bf16lo(l);
    x = bf16hi(h) + bf16hi(l);
  }
};

// Decay a_t of one step from its recurrence-gate pre-activation (same arithmetic as the forward).
__device__ __forceinline__ float decay_of(float pa, float kd) {
  return 1.0f + expm1_nonpos(kd * fast_sigmoid(pa));
}

// ---- pass 1: chunk maps --------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kBwdThreads) void bwd_summary(
    const typename PrePair<T>::type *__restrict__ pre, const T *__restrict__ dy,
    const float *__restrict__ Lambda, float2 *__restrict__ sums, int B, int Tn, int D, int nC) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * kBwdThreads + threadIdx.x;
  if (idx >= static_cast<size_t>(B) * D) return;
  const int b = static_cast<int>(idx / D);
  const int d = static_cast<int>(idx % D);
  const int c = blockIdx.y;
  const int s = c * kBwdChunk;
  const int e = min(s + kBwdChunk, Tn);
  const float kd = decay_coeff(Lambda[d]);
  const size_t base = static_cast<size_t>(b) * Tn * D + d;
  float P = 1.0f, g = 0.0f;
  for (int t0 = e - 1; t0 >= s; t0 -= 8) {
    float pa[8], dv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 - u;
      if (t >= s) {
        pa[u] = PrePair<T>::pa(pre[base + static_cast<size_t>(t) * D]);
        dv[u] = Elem<T>::load(dy, base + static_cast<size_t>(t) * D);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (t0 - u >= s) {
        const float a = decay_of(pa[u], kd);
        g = a * (dv[u] + g);
        P *= a;
      }
    }
  }
  sums[(static_cast<size_t>(b) * nC + c) * D + d] = make_float2(P, g);
}

// ---- pass 2: carries across chunks, right to left ------------------------------------------
__global__ __launch_bounds__(kBwdThreads) void bwd_carry(const float2 *__restrict__ sums,
                                                         const float *__restrict__ dh_T,
                                                         float *__restrict__ carry,
                                                         float *__restrict__ dh0, int B, int D,
                                                         int nC) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * kBwdThreads + threadIdx.x;
  if (idx >= static_cast<size_t>(B) * D) return;
  const int b = static_cast<int>(idx / D);
  const int d = static_cast<int>(idx % D);
  float g = dh_T ? dh_T[idx] : 0.0f;
  const size_t row = static_cast<size_t>(b) * nC;
  for (int c0 = nC - 1; c0 >= 0; c0 -= 8) {
    float2 sm[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c0 - u >= 0) sm[u] = sums[(row + c0 - u) * D + d];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (c0 - u >= 0) {
        carry[(row + c0 - u) * D + d] = g;
        g = fmaf(sm[u].x, g, sm[u].y);
      }
    }
  }
  if (dh0) dh0[idx] = g;
}

// ---- pass 3: per-element gradients ----------------------------------------------------------
// part: [3][B * nC][D] partial sums of dpa, dpx and r dz over each chunk.
template <typename T>
__global__ __launch_bounds__(kBwdThreads) void bwd_emit(
    const T *__restrict__ x, const typename PrePair<T>::type *__restrict__ pre,
    const T *__restrict__ y, const T *__restrict__ dy, const float *__restrict__ h0,
    const T *__restrict__ conv_w, const float *__restrict__ Lambda,
    const float *__restrict__ carry, typename DPair<T>::type *__restrict__ dpre,
    typename DPair<T>::type *__restrict__ dlo, float *__restrict__ dxc, float *__restrict__ part,
    int B, int Tn, int D, int nC) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * kBwdThreads + threadIdx.x;
  if (idx >= static_cast<size_t>(B) * D) return;
  const int b = static_cast<int>(idx / D);
  const int d = static_cast<int>(idx % D);
  const int c = blockIdx.y;
  const int s = c * kBwdChunk;
  const int e = min(s + kBwdChunk, Tn);
  float w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = Elem<T>::load(conv_w, static_cast<size_t>(j) * D + d);
  const float kd = decay_coeff(Lambda[d]);
  const size_t base = static_cast<size_t>(b) * Tn * D + d;
  const float hinit = h0 ? h0[idx] : 0.0f;
  // xw[j] = x[t - 3 + j] for the current t (zero before the sequence start)
  float xw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = e - 1 - 3 + j;
    xw[j] = q >= 0 ? Elem<T>::load(x, base + static_cast<size_t>(q) * D) : 0.0f;
  }
  float g = carry[(static_cast<size_t>(b) * nC + c) * D + d];
  float s_pa = 0.0f, s_px = 0.0f, s_rdz = 0.0f;
  for (int t0 = e - 1; t0 >= s; t0 -= 8) {
    typename PrePair<T>::type pp[8];
    float dv[8], hp[8], xn[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 - u;
      if (t >= s) {
        const size_t o = base + static_cast<size_t>(t) * D;
        pp[u] = pre[o];
        dv[u] = Elem<T>::load(dy, o);
        hp[u] = t > 0 ? Elem<T>::load(y, o - D) : hinit;
        xn[u] = t >= 4 ? Elem<T>::load(x, o - 4 * static_cast<size_t>(D)) : 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 - u;
      if (t >= s) {
        const float xc = fmaf(w[3], xw[3], fmaf(w[2], xw[2], fmaf(w[1], xw[1], w[0] * xw[0])));
        const float r = fast_sigmoid(PrePair<T>::pa(pp[u]));
        const float ig = fast_sigmoid(PrePair<T>::px(pp[u]));
        const float em = expm1_nonpos(kd * r);
        const float a = 1.0f + em;
        const float m = __builtin_amdgcn_sqrtf(-em * (2.0f + em));
        const float delta = dv[u] + g;
        const float dm = delta * ig * xc;
        const float di = delta * m * xc;
        float dz = delta * hp[u] * a;
        if (m > 0.0f) dz -= dm * (a * a / m);
        const float dpa = kd * dz * (r * (1.0f - r));
        const float dpx = di * (ig * (1.0f - ig));
        const size_t o = base + static_cast<size_t>(t) * D;
        DPair<T>::put(dpre, dlo, o, dpa, dpx);
        dxc[o] = delta * m * ig;
        s_pa += dpa;
        s_px += dpx;
        s_rdz = fmaf(r, dz, s_rdz);
        g = a * delta;
        xw[3] = xw[2];
        xw[2] = xw[1];
        xw[1] = xw[0];
        xw[0] = xn[u];
      }
    }
  }
  const size_t P = static_cast<size_t>(B) * nC * D;
  const size_t pidx = (static_cast<size_t>(b) * nC + c) * D + d;
  part[pidx] = s_pa;
  part[P + pidx] = s_px;
  part[2 * P + pidx] = s_rdz;
}

// ---- 4a: dxc += [dpa dpx] [W_a ; W_x] on MFMA (bf16, Dh in {32, 64, 128, 256}) -------------
// wti[g][i][2o + q] = W_q[g][o][i] (q = 0: W_a, 1: W_x): the weights transposed and interleaved so
// that the contraction index k = 2o + q matches the (dpa, dpx) pair layout of dpre.
__global__ void wt_prep(const bf16_t *__restrict__ W_a, const bf16_t *__restrict__ W_x,
                        bf16_t *__restrict__ wti, int H, int Dh) {
  const size_t n = static_cast<size_t>(H) * Dh * 2 * Dh;
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int k = static_cast<int>(idx % (2 * Dh));
  const size_t gi = idx / (2 * Dh);
  const int i = static_cast<int>(gi % Dh);
  const int g = static_cast<int>(gi / Dh);
  const int o = k >> 1;
  const bf16_t *W = (k & 1) ? W_x : W_a;
  wti[idx] = W[(static_cast<size_t>(g) * Dh + o) * Dh + i];
}

template <int DH>
__global__ __launch_bounds__(kThreads) void dxc_mfma(const uint32_t *__restrict__ dpre,
                                                     const bf16_t *__restrict__ wti,
                                                     float *__restrict__ dxc, int Tn, int D) {
  typedef GateTile<DH> C;
  constexpr int K = 2 * DH;
  constexpr int kLd = K + 8;  // LDS row stride in bf16 (16 B pad)
  __shared__ __attribute__((aligned(16))) bf16_t lds_a[kTileRows * kLd];
  const int t0 = blockIdx.x * kTileRows;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  // A tile: rows t0..t0+63 of this head's K = 2 DH bf16 (DH pairs), zero past T.
  {
    constexpr int kChunks = K / 8;  // 16-byte chunks per row
    for (int q = tid; q < kTileRows * kChunks; q += kThreads) {
      const int r = q / kChunks, ch = q % kChunks;
      const int t = t0 + r;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (t < Tn)
        v = *reinterpret_cast<const u32x4_t *>(
            dpre + (static_cast<size_t>(b) * Tn + t) * D + static_cast<size_t>(g) * DH + ch * 4);
      *reinterpret_cast<u32x4_t *>(lds_a + r * kLd + ch * 8) = v;
    }
  }
  __syncthreads();
  const int w = tid >> 6;
  const int lane = tid & 63;
  int g0, r0;
  bool active;
  C::assign(w, g0, r0, active);
  if (!active) return;
  const int lrow = lane & 31;
  const int khalf = (lane >> 5) * 8;
  const bf16_t *wg = wti + static_cast<size_t>(g) * DH * K;
  f32x16_t acc[C::kGPW][C::kRPW];
#pragma unroll
  for (int gi = 0; gi < C::kGPW; ++gi)
#pragma unroll
    for (int ri = 0; ri < C::kRPW; ++ri) acc[gi][ri] = f32x16_t{};
#pragma unroll 2
  for (int k0 = 0; k0 < K; k0 += 16) {
    bf16x8_t af[C::kRPW], bfr[C::kGPW];
#pragma unroll
    for (int ri = 0; ri < C::kRPW; ++ri)
      af[ri] = load_bf16x8(lds_a + ((r0 + ri) * 32 + lrow) * kLd + k0 + khalf);
#pragma unroll
    for (int gi = 0; gi < C::kGPW; ++gi)
      bfr[gi] = load_bf16x8(wg + static_cast<size_t>((g0 + gi) * 32 + lrow) * K + k0 + khalf);
#pragma unroll
    for (int gi = 0; gi < C::kGPW; ++gi)
#pragma unroll
      for (int ri = 0; ri < C::kRPW; ++ri)
        acc[gi][ri] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ri], bfr[gi], acc[gi][ri], 0, 0, 0);
  }
#pragma unroll
  for (int gi = 0; gi < C::kGPW; ++gi) {
    const int d = g * DH + (g0 + gi) * 32 + lrow;
#pragma unroll
    for (int ri = 0; ri < C::kRPW; ++ri)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int t = t0 + C::acc_row(r0 + ri, j, lane);
        if (t < Tn) {
          float *p = dxc + (static_cast<size_t>(b) * Tn + t) * D + d;
          *p += acc[gi][ri][j];
        }
      }
  }
}

// ---- 4b: the same on the vector ALU (fp32, or bf16 with other head sizes) -------------------
constexpr int kBwdValuRows = 16;

template <typename T>
__global__ __launch_bounds__(256) void dxc_valu(const typename DPair<T>::type *__restrict__ dpre,
                                                const typename DPair<T>::type *__restrict__ dlo,
                                                const T *__restrict__ W_a,
                                                const T *__restrict__ W_x, float *__restrict__ dxc,
                                                int Tn, int D, int Dh) {
  __shared__ float sa[kBwdValuRows * 256], sx[kBwdValuRows * 256];
  const int t0 = blockIdx.x * kBwdValuRows;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  for (int q = threadIdx.x; q < kBwdValuRows * Dh; q += blockDim.x) {
    const int r = q / Dh, o = q % Dh;
    const int t = t0 + r;
    float va = 0.0f, vx = 0.0f;
    if (t < Tn)
      DPair<T>::get(dpre, dlo,
                    (static_cast<size_t>(b) * Tn + t) * D + static_cast<size_t>(g) * Dh + o, va, vx);
    sa[r * Dh + o] = va;
    sx[r * Dh + o] = vx;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < kBwdValuRows * Dh; q += blockDim.x) {
    const int r = q / Dh, i = q % Dh;
    const int t = t0 + r;
    if (t >= Tn) continue;
    const size_t wb = static_cast<size_t>(g) * Dh * Dh + i;
    float acc = 0.0f;
    for (int o = 0; o < Dh; ++o) {
      acc = fmaf(sa[r * Dh + o], Elem<T>::load(W_a, wb + static_cast<size_t>(o) * Dh), acc);
      acc = fmaf(sx[r * Dh + o], Elem<T>::load(W_x, wb + static_cast<size_t>(o) * Dh), acc);
    }
    dxc[(static_cast<size_t>(b) * Tn + t) * D + static_cast<size_t>(g) * Dh + i] += acc;
  }
}

// ---- 5: conv backward -----------------------------------------------------------------------
// pcw: [B * nC][4][D] partial sums of dconv_w over each chunk.
template <typename T>
__global__ __launch_bounds__(kBwdThreads) void conv_bwd(const T *__restrict__ x,
                                                        const float *__restrict__ dxc,
                                                        const T *__restrict__ conv_w,
                                                        T *__restrict__ dx,
                                                        float *__restrict__ pcw, int B, int Tn,
                                                        int D, int nC) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * kBwdThreads + threadIdx.x;
  if (idx >= static_cast<size_t>(B) * D) return;
  const int b = static_cast<int>(idx / D);
  const int d = static_cast<int>(idx % D);
  const int c = blockIdx.y;
  const int s = c * kBwdChunk;
  const int e = min(s + kBwdChunk, Tn);
  float w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = Elem<T>::load(conv_w, static_cast<size_t>(j) * D + d);
  const size_t base = static_cast<size_t>(b) * Tn * D + d;
  // gw[k] = dxc[t + k] (zero at or past T); xw[j] = x[t - 3 + j] (zero before 0)
  float gw[4], xw[4];
#pragma unroll
  for (int k = 0; k < 3; ++k)
    gw[k + 1] = s + k < Tn ? dxc[base + static_cast<size_t>(s + k) * D] : 0.0f;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int q = s - 3 + j;
    xw[j + 1] = q >= 0 ? Elem<T>::load(x, base + static_cast<size_t>(q) * D) : 0.0f;
  }
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int t0 = s; t0 < e; t0 += 8) {
    float gn[8], xn[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 + u;
      if (t < e) {
        gn[u] = t + 3 < Tn ? dxc[base + static_cast<size_t>(t + 3) * D] : 0.0f;
        xn[u] = Elem<T>::load(x, base + static_cast<size_t>(t) * D);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 + u;
      if (t < e) {
        gw[0] = gw[1];
        gw[1] = gw[2];
        gw[2] = gw[3];
        gw[3] = gn[u];
        xw[0] = xw[1];
        xw[1] = xw[2];
        xw[2] = xw[3];
        xw[3] = xn[u];
        // dx[t] = sum_j w[j] dxc[t + 3 - j]
        const float v = fmaf(w[0], gw[3], fmaf(w[1], gw[2], fmaf(w[2], gw[1], w[3] * gw[0])));
        Elem<T>::store(dx, base + static_cast<size_t>(t) * D, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = fmaf(gw[0], xw[j], acc[j]);
      }
    }
  }
  const size_t prow = (static_cast<size_t>(b) * nC + c) * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) pcw[(prow + j) * D + d] = acc[j];
}

// ---- 6a: dW partials on MFMA (bf16, Dh in {128, 256}) ---------------------------------------
// Output tile 128 (m = 2o + q) x 128 (i) of head g, contraction over the rows [kb, ke) of the
// flattened (b, t) index; 4 waves in a 2 x 2 grid, each 64 x 64 = 2 x 2 MFMA tiles. Per step of 64
// rows, dp and the conv output xc (recomputed from x in fp32) are written to LDS transposed, k
// contiguous, so both MFMA operands read 16 B per lane.
// Precision: with both operands rounded to bf16 a dW element errs by up to 2^-9 of its largest
// terms, and the gate gradients are heavy tailed (dz carries 1/m), so single elements of dW miss
// by a few percent of the tensor's rms. Each operand is therefore split into bf16 hi + lo and
// the product taken as hi*hi + lo*hi + hi*lo (the lo*lo term is below 2^-16), three MFMAs per
// tile step with fp32 accumulation.
// pw: [S][H][2 Dh][Dh] fp32.
constexpr int kDwRows = 64;
constexpr int kDwLd = kDwRows + 8;  // bf16 per LDS row (16 B pad)

template <int DH>
__global__ __launch_bounds__(256) void dw_mfma(const bf16_t *__restrict__ x,
                                               const uint32_t *__restrict__ dpre,
                                               const uint32_t *__restrict__ dlo,
                                               const bf16_t *__restrict__ conv_w,
                                               float *__restrict__ pw, int Tn, int D, int H,
                                               long long rows, long long rows_per_split) {
  static_assert(DH == 128 || DH == 256, "dW MFMA tile needs Dh in {128, 256}");
  constexpr int kMt = 2 * DH / 128;
  __shared__ __attribute__((aligned(16))) bf16_t la[2][128 * kDwLd];  // [hi, lo][m][k]
  __shared__ __attribute__((aligned(16))) bf16_t lb[2][128 * kDwLd];  // [hi, lo][i][k]
  const int mt = blockIdx.x % kMt;
  const int nt = blockIdx.x / kMt;
  const int g = blockIdx.y;
  const int sp = blockIdx.z;
  const long long kb = static_cast<long long>(sp) * rows_per_split;
  const long long ke = min(kb + rows_per_split, rows);
  const int tid = threadIdx.x;
  // loader role: 4 consecutive rows (q) x 8 consecutive columns (j)
  const int lq = tid & 15;   // row quad 0..15
  const int lj = tid >> 4;   // column octet 0..15
  // A columns m = mt*128 + 8 lj .. +7, i.e. the pairs o = (mt*128 + 8 lj)/2 .. +3 of this head
  const size_t a_col = static_cast<size_t>(g) * DH + (mt * 128 + 8 * lj) / 2;  // uint32 pairs
  const size_t b_col = static_cast<size_t>(g) * DH + nt * 128 + 8 * lj;       // bf16 channels
  float cw[4][8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(conv_w + static_cast<size_t>(j) * D + b_col);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      cw[j][2 * h] = bf16lo(v[h]);
      cw[j][2 * h + 1] = bf16hi(v[h]);
    }
  }
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int wm = (w & 1) * 64, wn = (w >> 1) * 64;
  const int lrow = lane & 31;
  const int khalf = (lane >> 5) * 8;
  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[a][c] = f32x16_t{};

  for (long long k0 = kb; k0 < ke; k0 += kDwRows) {
    // ---- load; conv in fp32
    uint32_t av[2][4][4];  // [hi, lo][row u][pair h]: 4 pairs = 8 values of m
    float xcv[4][8];       // [row u][column]
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long long rr = k0 + 4 * lq + u;
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) xcv[u][cc] = 0.0f;
      if (rr < ke) {
        const int bb = static_cast<int>(rr / Tn);
        const int t = static_cast<int>(rr % Tn);
        const size_t rowoff = (static_cast<size_t>(bb) * Tn + t) * D;
        const u32x4_t vh = *reinterpret_cast<const u32x4_t *>(dpre + rowoff + a_col);
        const u32x4_t vl = *reinterpret_cast<const u32x4_t *>(dlo + rowoff + a_col);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          av[0][u][h] = vh[h];
          av[1][u][h] = vl[h];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int ts = t - 3 + j;
          if (ts >= 0) {
            const u32x4_t xv = *reinterpret_cast<const u32x4_t *>(
                x + (static_cast<size_t>(bb) * Tn + ts) * D + b_col);
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              xcv[u][2 * h] = fmaf(cw[j][2 * h], bf16lo(xv[h]), xcv[u][2 * h]);
              xcv[u][2 * h + 1] = fmaf(cw[j][2 * h + 1], bf16hi(xv[h]), xcv[u][2 * h + 1]);
            }
          }
        }
      } else {
#pragma unroll
        for (int h = 0; h < 4; ++h) av[0][u][h] = av[1][u][h] = 0u;
      }
    }
    __syncthreads();  // the previous step's MFMA reads are done
    // ---- transpose into LDS: row m (or i), 4 consecutive k per 8-byte store
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const int h = cc >> 1;
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        const uint32_t(&q)[4][4] = av[part];
        uint32_t a01, a23;
        if (cc & 1) {  // m odd: the dpx halves
          a01 = (q[0][h] >> 16) | (q[1][h] & 0xffff0000u);
          a23 = (q[2][h] >> 16) | (q[3][h] & 0xffff0000u);
        } else {       // m even: the dpa halves
          a01 = (q[0][h] & 0xffffu) | (q[1][h] << 16);
          a23 = (q[2][h] & 0xffffu) | (q[3][h] << 16);
        }
        *reinterpret_cast<uint2 *>(&la[part][(8 * lj + cc) * kDwLd + 4 * lq]) = make_uint2(a01, a23);
      }
      const uint32_t h01 = pack_bf16x2(xcv[0][cc], xcv[1][cc]);
      const uint32_t h23 = pack_bf16x2(xcv[2][cc], xcv[3][cc]);
      const uint32_t l01 = pack_bf16x2(xcv[0][cc] - bf16lo(h01), xcv[1][cc] - bf16hi(h01));
      const uint32_t l23 = pack_bf16x2(xcv[2][cc] - bf16lo(h23), xcv[3][cc] - bf16hi(h23));
      *reinterpret_cast<uint2 *>(&lb[0][(8 * lj + cc) * kDwLd + 4 * lq]) = make_uint2(h01, h23);
      *reinterpret_cast<uint2 *>(&lb[1][(8 * lj + cc) * kDwLd + 4 * lq]) = make_uint2(l01, l23);
    }
    __syncthreads();
    // ---- MFMA over the 64 rows: hi*hi + lo*hi + hi*lo
#pragma unroll
    for (int kk = 0; kk < kDwRows; kk += 16) {
      bf16x8_t af[2][2], bfr[2][2];  // [hi, lo][tile]
#pragma unroll
      for (int part = 0; part < 2; ++part)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          af[part][a] = load_bf16x8(&la[part][(wm + a * 32 + lrow) * kDwLd + kk + khalf]);
          bfr[part][a] = load_bf16x8(&lb[part][(wn + a * 32 + lrow) * kDwLd + kk + khalf]);
        }
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int c = 0; c < 2; ++c)
            acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[p == 1][a], bfr[p == 2][c],
                                                                acc[a][c], 0, 0, 0);
    }
  }
  // ---- partial out: pw[sp][g][m][i]
  float *dst = pw + (static_cast<size_t>(sp) * H + g) * (2 * DH) * DH;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int m = mt * 128 + wm + a * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
        const int i = nt * 128 + wn + c * 32 + lrow;
        dst[static_cast<size_t>(m) * DH + i] = acc[a][c][j];
      }
}

// ---- 6b: dW partials on the vector ALU ------------------------------------------------------
// Output tile 64 (m) x 64 (i); 256 threads, each 4 x 4. Rows in steps of 16 staged in LDS.
template <typename T>
__global__ __launch_bounds__(256) void dw_valu(const T *__restrict__ x,
                                               const typename DPair<T>::type *__restrict__ dpre,
                                               const typename DPair<T>::type *__restrict__ dlo,
                                               const T *__restrict__ conv_w,
                                               float *__restrict__ pw, int Tn, int D, int H,
                                               int Dh, long long rows, long long rows_per_split) {
  __shared__ float sa[16][64], sb[16][64];
  const int nMt = (2 * Dh + 63) / 64;
  const int mt = blockIdx.x % nMt;
  const int nt = blockIdx.x / nMt;
  const int g = blockIdx.y;
  const int sp = blockIdx.z;
  const long long kb = static_cast<long long>(sp) * rows_per_split;
  const long long ke = min(kb + rows_per_split, rows);
  const int tid = threadIdx.x;
  const int tm = (tid & 15) * 4, tn = (tid >> 4) * 4;
  float acc[4][4] = {};
  for (long long k0 = kb; k0 < ke; k0 += 16) {
    for (int q = tid; q < 16 * 64; q += 256) {
      const int r = q / 64, col = q % 64;
      const long long rr = k0 + r;
      float va = 0.0f, vb = 0.0f;
      if (rr < ke) {
        const int bb = static_cast<int>(rr / Tn);
        const int t = static_cast<int>(rr % Tn);
        const size_t rowoff = (static_cast<size_t>(bb) * Tn + t) * D;
        const int m = mt * 64 + col;
        if (m < 2 * Dh) {
          float pa_, px_;
          DPair<T>::get(dpre, dlo, rowoff + static_cast<size_t>(g) * Dh + (m >> 1), pa_, px_);
          va = (m & 1) ? px_ : pa_;
        }
        const int i = nt * 64 + col;
        if (i < Dh) {
          const size_t dd = static_cast<size_t>(g) * Dh + i;
          for (int j = 0; j < 4; ++j) {
            const int ts = t - 3 + j;
            if (ts >= 0)
              vb = fmaf(Elem<T>::load(conv_w, static_cast<size_t>(j) * D + dd),
                        Elem<T>::load(x, (static_cast<size_t>(bb) * Tn + ts) * D + dd), vb);
          }
        }
      }
      sa[r][col] = va;
      sb[r][col] = vb;
    }
    __syncthreads();
#pragma unroll 4
    for (int r = 0; r < 16; ++r) {
      float av[4], bv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        av[u] = sa[r][tm + u];
        bv[u] = sb[r][tn + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(av[u], bv[v], acc[u][v]);
    }
    __syncthreads();
  }
  float *dst = pw + (static_cast<size_t>(sp) * H + g) * (2 * Dh) * Dh;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int m = mt * 64 + tm + u;
    if (m >= 2 * Dh) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = nt * 64 + tn + v;
      if (i < Dh) dst[static_cast<size_t>(m) * Dh + i] = acc[u][v];
    }
  }
}

// ---- 7: fixed-order reduction of the partials ----------------------------------------------
// Index ranges: [0, D) -> db_a, db_x, dLambda; [D, 5D) -> dconv_w; then 2 H Dh^2 -> dW_a, dW_x.
__global__ __launch_bounds__(256) void bwd_reduce(const float *__restrict__ part,
                                                  const float *__restrict__ pcw,
                                                  const float *__restrict__ pw,
                                                  const float *__restrict__ Lambda,
                                                  float *__restrict__ db_a,
                                                  float *__restrict__ db_x,
                                                  float *__restrict__ dLambda,
                                                  float *__restrict__ dconv_w,
                                                  float *__restrict__ dW_a,
                                                  float *__restrict__ dW_x, int D, int H,
                                                  int Dh, int P, int S) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const size_t nW = static_cast<size_t>(H) * Dh * Dh;
  if (idx < static_cast<size_t>(D)) {
    const size_t Pd = static_cast<size_t>(P) * D;
    float sa = 0.0f, sx = 0.0f, sr = 0.0f;
    for (int p = 0; p < P; ++p) {
      sa += part[static_cast<size_t>(p) * D + idx];
      sx += part[Pd + static_cast<size_t>(p) * D + idx];
      sr += part[2 * Pd + static_cast<size_t>(p) * D + idx];
    }
    db_a[idx] = sa;
    db_x[idx] = sx;
    // d softplus(-L)/dL = -sigmoid(-L); dLambda = 8 sigmoid(-L) sum r dz
    const float sig = 1.0f / (1.0f + expf(Lambda[idx]));
    dLambda[idx] = kGateC * sig * sr;
  } else if (idx < static_cast<size_t>(5) * D) {
    const size_t q = idx - D;  // = j * D + d
    const int j = static_cast<int>(q / D);
    const int d = static_cast<int>(q % D);
    float sacc = 0.0f;
    for (int p = 0; p < P; ++p) sacc += pcw[(static_cast<size_t>(p) * 4 + j) * D + d];
    dconv_w[q] = sacc;
  } else if (idx < static_cast<size_t>(5) * D + 2 * nW) {
    const size_t q = idx - static_cast<size_t>(5) * D;  // = gate * nW + (g Dh + o) Dh + i
    const int gate = static_cast<int>(q / nW);
    const size_t r = q % nW;
    const int i = static_cast<int>(r % Dh);
    const size_t go = r / Dh;
    const int o = static_cast<int>(go % Dh);
    const int g = static_cast<int>(go / Dh);
    const size_t src = (static_cast<size_t>(g) * 2 * Dh + 2 * o + gate) * Dh + i;
    const size_t stride = static_cast<size_t>(H) * 2 * Dh * Dh;
    float sacc = 0.0f;
    for (int s = 0; s < S; ++s) sacc += pw[static_cast<size_t>(s) * stride + src];
    (gate ? dW_x : dW_a)[r] = sacc;
  }
}

// ---- host side ------------------------------------------------------------------------------
BwdLayout backward_layout(int B, int T, int D, int H, int io) {
  BwdLayout L;
  const int Dh = D / H;
  L.nC = (T + kBwdChunk - 1) / kBwdChunk;
  const long long rows = static_cast<long long>(B) * T;
  L.mfma_dxc = io == kBF16 && (Dh == 32 || Dh == 64 || Dh == 128 || Dh == 256);
  L.mfma_dw = io == kBF16 && (Dh == 128 || Dh == 256);
  const int tiles = L.mfma_dw ? (2 * Dh / 128) * (Dh / 128)
                              : ((2 * Dh + 63) / 64) * ((Dh + 63) / 64);
  const int step = L.mfma_dw ? kDwRows : 16;
  const long long steps = (rows + step - 1) / step;
  // enough row splits for about 1024 workgroups, each at least one step of rows
  long long S = (1024 + static_cast<long long>(tiles) * H - 1) / (static_cast<long long>(tiles) * H);
  S = std::max<long long>(1, std::min<long long>(S, std::min<long long>(steps, 65535)));
  L.rows_per_split = (steps + S - 1) / S * step;
  L.S = static_cast<int>((rows + L.rows_per_split - 1) / L.rows_per_split);
  const size_t n = static_cast<size_t>(B) * T * D;
  const size_t pairb = io == kBF16 ? 4 : 8;
  const size_t P = static_cast<size_t>(B) * L.nC;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t r = off;
    off += (bytes + 255) / 256 * 256;
    return r;
  };
  L.o_pre = take(n * pairb);
  L.o_dpre = take(n * pairb);
  L.o_dlo = take(io == kBF16 ? n * 4 : 0);
  L.o_dxc = take(n * sizeof(float));
  L.o_sums = take(P * D * sizeof(float2));
  L.o_carry = take(P * D * sizeof(float));
  L.o_part = take(3 * P * D * sizeof(float));
  L.o_pcw = take(4 * P * D * sizeof(float));
  L.o_pw = take(static_cast<size_t>(L.S) * H * 2 * Dh * Dh * sizeof(float));
  L.o_wti = take(L.mfma_dxc ? static_cast<size_t>(H) * Dh * 2 * Dh * sizeof(bf16_t) : 0);
  L.total = off;
  return L;
}

template <typename T>
static hipError_t run_backward(const T *x, const T *conv_w, const T *W_a, const float *b_a,
                               const T *W_x, const float *b_x, const float *Lambda,
                               const float *h0, const T *y, const T *dy, const float *dh_T, T *dx,
                               float *dconv_w, float *dW_a, float *db_a, float *dW_x,
                               float *db_x, float *dLambda, float *dh0, int B, int Tn, int D,
                               int H, const BwdLayout &L, char *ws, hipStream_t s) {
  const int io = sizeof(T) == 2 ? kBF16 : kF32;
  const int Dh = D / H;
  typedef typename PrePair<T>::type PP;
  typedef typename DPair<T>::type DP;
  PP *pre = reinterpret_cast<PP *>(ws + L.o_pre);
  DP *dpre = reinterpret_cast<DP *>(ws + L.o_dpre);
  DP *dlo = sizeof(T) == 2 ? reinterpret_cast<DP *>(ws + L.o_dlo) : nullptr;
  float *dxc = reinterpret_cast<float *>(ws + L.o_dxc);
  float2 *sums = reinterpret_cast<float2 *>(ws + L.o_sums);
  float *carry = reinterpret_cast<float *>(ws + L.o_carry);
  float *part = reinterpret_cast<float *>(ws + L.o_part);
  float *pcw = reinterpret_cast<float *>(ws + L.o_pcw);
  float *pw = reinterpret_cast<float *>(ws + L.o_pw);
  // pre-activations recomputed with the conv output split into bf16 hi + lo: the gradients
  // amplify pre-activation errors (through r (1 - r) and 1/m), so the backward does not reuse
  // the forward's bf16-operand rounding
  hipError_t e = launch_gates(x, conv_w, W_a, b_a, W_x, b_x, pre, B, Tn, D, H, io, s, true);
  if (e != hipSuccess) return e;
  const size_t lanes = static_cast<size_t>(B) * D;
  const dim3 lgrid(static_cast<unsigned>((lanes + kBwdThreads - 1) / kBwdThreads), L.nC);
  const unsigned lblocks = static_cast<unsigned>((lanes + kBwdThreads - 1) / kBwdThreads);
  bwd_summary<T><<<lgrid, kBwdThreads, 0, s>>>(pre, dy, Lambda, sums, B, Tn, D, L.nC);
  bwd_carry<<<lblocks, kBwdThreads, 0, s>>>(sums, dh_T, carry, dh0, B, D, L.nC);
  bwd_emit<T><<<lgrid, kBwdThreads, 0, s>>>(x, pre, y, dy, h0, conv_w, Lambda, carry, dpre, dlo,
                                            dxc, part, B, Tn, D, L.nC);
  if constexpr (sizeof(T) == 2) {
    if (L.mfma_dxc) {
      bf16_t *wti = reinterpret_cast<bf16_t *>(ws + L.o_wti);
      const size_t nw = static_cast<size_t>(H) * Dh * 2 * Dh;
      wt_prep<<<static_cast<unsigned>((nw + 255) / 256), 256, 0, s>>>(W_a, W_x, wti, H, Dh);
      const dim3 grid((Tn + kTileRows - 1) / kTileRows, H, B);
      switch (Dh) {
        case 32: dxc_mfma<32><<<grid, kThreads, 0, s>>>(dpre, wti, dxc, Tn, D); break;
        case 64: dxc_mfma<64><<<grid, kThreads, 0, s>>>(dpre, wti, dxc, Tn, D); break;
        case 128: dxc_mfma<128><<<grid, kThreads, 0, s>>>(dpre, wti, dxc, Tn, D); break;
        case 256: dxc_mfma<256><<<grid, kThreads, 0, s>>>(dpre, wti, dxc, Tn, D); break;
        default: return hipErrorInvalidValue;
      }
    }
  }
  if (!L.mfma_dxc) {
    const dim3 grid((Tn + kBwdValuRows - 1) / kBwdValuRows, H, B);
    dxc_valu<T><<<grid, 256, 0, s>>>(dpre, dlo, W_a, W_x, dxc, Tn, D, Dh);
  }
  conv_bwd<T><<<lgrid, kBwdThreads, 0, s>>>(x, dxc, conv_w, dx, pcw, B, Tn, D, L.nC);
  const long long rows = static_cast<long long>(B) * Tn;
  if constexpr (sizeof(T) == 2) {
    if (L.mfma_dw) {
      const dim3 grid((2 * Dh / 128) * (Dh / 128), H, L.S);
      if (Dh == 256)
        dw_mfma<256><<<grid, 256, 0, s>>>(x, dpre, dlo, conv_w, pw, Tn, D, H, rows,
                                          L.rows_per_split);
      else
        dw_mfma<128><<<grid, 256, 0, s>>>(x, dpre, dlo, conv_w, pw, Tn, D, H, rows,
                                          L.rows_per_split);
    }
  }
  if (!L.mfma_dw) {
    const dim3 grid(((2 * Dh + 63) / 64) * ((Dh + 63) / 64), H, L.S);
    dw_valu<T><<<grid, 256, 0, s>>>(x, dpre, dlo, conv_w, pw, Tn, D, H, Dh, rows,
                                     L.rows_per_split);
  }
  const size_t nred = static_cast<size_t>(5) * D + 2 * static_cast<size_t>(H) * Dh * Dh;
  bwd_reduce<<<static_cast<unsigned>((nred + 255) / 256), 256, 0, s>>>(
      part, pcw, pw, Lambda, db_a, db_x, dLambda, dconv_w, dW_a, dW_x, D, H, Dh, B * L.nC, L.S);
  return hipGetLastError();
}

hipError_t launch_backward(const void *x, const void *conv_w, const void *W_a, const float *b_a,
                           const void *W_x, const float *b_x, const float *Lambda,
                           const float *h0, const void *y, const void *dy, const float *dh_T,
                           void *dx, float *dconv_w, float *dW_a, float *db_a, float *dW_x,
                           float *db_x, float *dLambda, float *dh0, int B, int T, int D, int H,
                           int io, void *workspace, hipStream_t s) {
  const BwdLayout L = backward_layout(B, T, D, H, io);
  char *ws = static_cast<char *>(workspace);
  if (io == kBF16)
    return run_backward<bf16_t>(
        static_cast<const bf16_t *>(x), static_cast<const bf16_t *>(conv_w),
        static_cast<const bf16_t *>(W_a), b_a, static_cast<const bf16_t *>(W_x), b_x, Lambda, h0,
        static_cast<const bf16_t *>(y), static_cast<const bf16_t *>(dy), dh_T,
        static_cast<bf16_t *>(dx), dconv_w, dW_a, db_a, dW_x, db_x, dLambda, dh0, B, T, D, H, L,
        ws, s);
  return run_backward<float>(
      static_cast<const float *>(x), static_cast<const float *>(conv_w),
      static_cast<const float *>(W_a), b_a, static_cast<const float *>(W_x), b_x, Lambda, h0,
      static_cast<const float *>(y), static_cast<const float *>(dy), dh_T,
      static_cast<float *>(dx), dconv_w, dW_a, db_a, dW_x, db_x, dLambda, dh0, B, T, D, H, L, ws,
      s);
}

}  // namespace rglru
