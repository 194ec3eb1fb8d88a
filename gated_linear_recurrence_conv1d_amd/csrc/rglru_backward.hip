// rglru_backward.hip -- gradients of the Conv1D(width 4) -> RG-LRU forward.
//
// The forward (the RG-LRU named by the Griffin paper page on docshare.wps.com, abstract and
// Introduction, with the equations the forward's header writes out; the gate that can discard
// the input and keep the history, Soham De's Griffin thread, tweet on adding a
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
//  4. dxc_mfma / dxc_valu: dxc += [dpa dpx] [W_a ; W_x] per head (fp16 MFMA or fp32 VALU).
//  5. conv_bwd: dx from dxc and conv_w; per-chunk partials of dconv_w.
//  6. dw_mfma / dw_valu: per head and row split, partial dW = dp^T xc with xc recomputed from x.
//  7. colsum: fixed-order sums of all partials (deterministic: no floating-point atomics).
#include <algorithm>

#include "rglru_launch.h"
#include "rglru_mfma.h"

namespace rglru {

constexpr int kBwdThreads = 256;

// (dpa, dpx) pair storage. fp32 I/O: one float2 (dpa first). bf16 I/O: the pair as two fp16
// (dpa in the low half): 11 significant bits, which the dW contraction needs (bf16's 8 left single
// elements of dW off by a few percent of the rms; see dw_mfma), in the 4 bytes of a bf16 pair.
// The gate gradients stay far inside fp16's range (|dp| < 65504) at the configurations measured
// here: they scale as delta * xc, the factor 1/m of dz being cancelled by r (1 - r).
template <typename T> struct DPair;
template <> struct DPair<float> {
  typedef float2 type;
  __device__ __forceinline__ static void put(type *p, size_t o, float a, float x) {
    p[o] = make_float2(a, x);
  }
  template <int CH>
  __device__ __forceinline__ static void put(type *p, size_t o, const float (&a)[CH],
                                             const float (&x)[CH]) {
    if constexpr (CH == 2)
      *reinterpret_cast<float4 *>(p + o) = make_float4(a[0], x[0], a[1], x[1]);
    else
      put(p, o, a[0], x[0]);
  }
  __device__ __forceinline__ static void get(const type *p, size_t o, float &a, float &x) {
    const float2 v = p[o];
    a = v.x;
    x = v.y;
  }
};
template <> struct DPair<bf16_t> {
  typedef uint32_t type;
  __device__ __forceinline__ static void put(type *p, size_t o, float a, float x) {
    p[o] = pack_f16x2(a, x);
  }
  template <int CH>
  __device__ __forceinline__ static void put(type *p, size_t o, const float (&a)[CH],
                                             const float (&x)[CH]) {
    if constexpr (CH == 2)
      *reinterpret_cast<uint2 *>(p + o) = make_uint2(pack_f16x2(a[0], x[0]), pack_f16x2(a[1], x[1]));
    else
      put(p, o, a[0], x[0]);
  }
  __device__ __forceinline__ static void get(const type *p, size_t o, float &a, float &x) {
    const uint32_t h = p[o];
    a = f16lo(h);
    x = f16hi(h);
  }
};

// Decay a_t of one step from its recurrence-gate pre-activation (same arithmetic as the forward).
__device__ __forceinline__ float decay_of(float pa, float kd) {
  return 1.0f + expm1_nonpos(kd * fast_sigmoid(pa));
}

// The lane kernels below (chunk maps, gradients, conv backward) give each lane CH = 1 or 2
// adjacent channels of one sequence, so that with CH = 2 every access moves twice the bytes per
// instruction. Loads and stores of CH consecutive elements of one row:
template <typename T, int CH> struct Lanes;
template <> struct Lanes<bf16_t, 1> {
  __device__ __forceinline__ static void load(const bf16_t *p, size_t i, float (&v)[1]) {
    v[0] = bf16_to_f32(p[i]);
  }
  __device__ __forceinline__ static void store(bf16_t *p, size_t i, const float (&v)[1]) {
    p[i] = f32_to_bf16(v[0]);
  }
};
template <> struct Lanes<bf16_t, 2> {
  __device__ __forceinline__ static void load(const bf16_t *p, size_t i, float (&v)[2]) {
    const uint32_t u = *reinterpret_cast<const uint32_t *>(p + i);
    v[0] = bf16lo(u);
    v[1] = bf16hi(u);
  }
  __device__ __forceinline__ static void store(bf16_t *p, size_t i, const float (&v)[2]) {
    *reinterpret_cast<uint32_t *>(p + i) = pack_bf16x2(v[0], v[1]);
  }
};
template <> struct Lanes<bf16_t, 4> {
  __device__ __forceinline__ static void load(const bf16_t *p, size_t i, float (&v)[4]) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p + i);
    v[0] = bf16lo(u.x);
    v[1] = bf16hi(u.x);
    v[2] = bf16lo(u.y);
    v[3] = bf16hi(u.y);
  }
  __device__ __forceinline__ static void store(bf16_t *p, size_t i, const float (&v)[4]) {
    *reinterpret_cast<uint2 *>(p + i) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
};
template <> struct Lanes<float, 1> {
  __device__ __forceinline__ static void load(const float *p, size_t i, float (&v)[1]) { v[0] = p[i]; }
  __device__ __forceinline__ static void store(float *p, size_t i, const float (&v)[1]) { p[i] = v[0]; }
};
template <> struct Lanes<float, 2> {
  __device__ __forceinline__ static void load(const float *p, size_t i, float (&v)[2]) {
    const float2 u = *reinterpret_cast<const float2 *>(p + i);
    v[0] = u.x;
    v[1] = u.y;
  }
  __device__ __forceinline__ static void store(float *p, size_t i, const float (&v)[2]) {
    *reinterpret_cast<float2 *>(p + i) = make_float2(v[0], v[1]);
  }
};
// Storage of dxc, the gradient of the conv output: fp32 for fp32 I/O; fp16 for bf16 I/O (2^-11
// of rounding, a quarter of the bf16 output's, in half the bytes: it is written and read back
// twice per element; its range is that of delta, far inside fp16's at the configurations measured
// here). One element (ld / st) or CH consecutive ones (load / store).
template <typename T, int CH = 1> struct DxcS;
template <int CH> struct DxcS<float, CH> {
  typedef float type;
  __device__ __forceinline__ static float ld(const type *p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void st(type *p, size_t i, float v) { p[i] = v; }
  __device__ __forceinline__ static void load(const type *p, size_t i, float (&v)[CH]) {
    Lanes<float, CH>::load(p, i, v);
  }
  __device__ __forceinline__ static void store(type *p, size_t i, const float (&v)[CH]) {
    Lanes<float, CH>::store(p, i, v);
  }
};
template <int CH> struct DxcS<bf16_t, CH> {
  typedef uint16_t type;
  __device__ __forceinline__ static float ld(const type *p, size_t i) {
    return f16lo(static_cast<uint32_t>(p[i]));
  }
  __device__ __forceinline__ static void st(type *p, size_t i, float v) {
    p[i] = static_cast<uint16_t>(pack_f16x2(v, 0.0f));
  }
  __device__ __forceinline__ static void load(const type *p, size_t i, float (&v)[CH]) {
    if constexpr (CH == 4) {
      const uint2 u = *reinterpret_cast<const uint2 *>(p + i);
      v[0] = f16lo(u.x);
      v[1] = f16hi(u.x);
      v[2] = f16lo(u.y);
      v[3] = f16hi(u.y);
    } else if constexpr (CH == 2) {
      const uint32_t u = *reinterpret_cast<const uint32_t *>(p + i);
      v[0] = f16lo(u);
      v[1] = f16hi(u);
    } else {
      v[0] = ld(p, i);
    }
  }
  __device__ __forceinline__ static void store(type *p, size_t i, const float (&v)[CH]) {
    if constexpr (CH == 2)
      *reinterpret_cast<uint32_t *>(p + i) = pack_f16x2(v[0], v[1]);
    else
      st(p, i, v[0]);
  }
};

// CH pre-activation pairs in their storage layout (PrePair) as one access.
template <typename T, int CH> struct PreLanes {
  typedef typename PrePair<T>::type P;
  struct alignas(sizeof(P) * CH) type {
    P v[CH];
  };
  __device__ __forceinline__ static type load(const P *p, size_t i) {
    return *reinterpret_cast<const type *>(p + i);
  }
};

// ---- pass 1: chunk maps --------------------------------------------------------------------
template <typename T, int CH>
__global__ __launch_bounds__(kBwdThreads) void bwd_summary(
    const typename PrePair<T>::type *__restrict__ pre, const T *__restrict__ dy,
    const float *__restrict__ Lambda, float2 *__restrict__ sums, int B, int Tn, int D, int nC) {
  const int DL = D / CH;  // lanes per sequence
  const size_t idx = static_cast<size_t>(blockIdx.x) * kBwdThreads + threadIdx.x;
  if (idx >= static_cast<size_t>(B) * DL) return;
  const int b = static_cast<int>(idx / DL);
  const int d0 = static_cast<int>(idx % DL) * CH;
  const int c = blockIdx.y;
  const int s = c * kBwdChunk;
  const int e = min(s + kBwdChunk, Tn);
  float kd[CH], P[CH], g[CH];
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    kd[k] = decay_coeff(Lambda[d0 + k]);
    P[k] = 1.0f;
    g[k] = 0.0f;
  }
  const size_t base = static_cast<size_t>(b) * Tn * D + d0;
  for (int t0 = e - 1; t0 >= s; t0 -= 8) {
    typename PreLanes<T, CH>::type pp[8];
    float dv[8][CH];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 - u;
      if (t >= s) {
        const size_t o = base + static_cast<size_t>(t) * D;
        pp[u] = PreLanes<T, CH>::load(pre, o);
        Lanes<T, CH>::load(dy, o, dv[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (t0 - u >= s) {
#pragma unroll
        for (int k = 0; k < CH; ++k) {
          const float a = decay_of(PrePair<T>::pa(pp[u].v[k]), kd[k]);
          g[k] = a * (dv[u][k] + g[k]);
          P[k] *= a;
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < CH; ++k)
    sums[(static_cast<size_t>(b) * nC + c) * D + d0 + k] = make_float2(P[k], g[k]);
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
template <typename T, int CH>
__global__ __launch_bounds__(kBwdThreads) void bwd_emit(
    const T *__restrict__ x, const typename PrePair<T>::type *__restrict__ pre,
    const T *__restrict__ y, const T *__restrict__ dy, const float *__restrict__ h0,
    const T *__restrict__ conv_w, const float *__restrict__ Lambda,
    const float *__restrict__ carry, typename DPair<T>::type *__restrict__ dpre,
    typename DxcS<T>::type *__restrict__ dxc, float *__restrict__ part,
    int B, int Tn, int D, int nC) {
  const int DL = D / CH;
  const size_t idx = static_cast<size_t>(blockIdx.x) * kBwdThreads + threadIdx.x;
  if (idx >= static_cast<size_t>(B) * DL) return;
  const int b = static_cast<int>(idx / DL);
  const int d0 = static_cast<int>(idx % DL) * CH;
  const int c = blockIdx.y;
  const int s = c * kBwdChunk;
  const int e = min(s + kBwdChunk, Tn);
  float w[4][CH];
#pragma unroll
  for (int j = 0; j < 4; ++j) Lanes<T, CH>::load(conv_w, static_cast<size_t>(j) * D + d0, w[j]);
  float kd[CH], hinit[CH], g[CH], s_pa[CH], s_px[CH], s_rdz[CH];
  const size_t cidx = (static_cast<size_t>(b) * nC + c) * D + d0;
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    kd[k] = decay_coeff(Lambda[d0 + k]);
    hinit[k] = h0 ? h0[static_cast<size_t>(b) * D + d0 + k] : 0.0f;
    g[k] = carry[cidx + k];
    s_pa[k] = s_px[k] = s_rdz[k] = 0.0f;
  }
  const size_t base = static_cast<size_t>(b) * Tn * D + d0;
  // xw[j] = x[t - 3 + j] for the current t (zero before the sequence start)
  float xw[4][CH];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = e - 1 - 3 + j;
    if (q >= 0) {
      Lanes<T, CH>::load(x, base + static_cast<size_t>(q) * D, xw[j]);
    } else {
#pragma unroll
      for (int k = 0; k < CH; ++k) xw[j][k] = 0.0f;
    }
  }
  // Groups of kG steps, double buffered: the loads of group i+1 are issued before group i's
  // arithmetic and stores, so that waiting for them never waits behind this group's stores
  // (loads and stores retire in issue order).
  constexpr int kG = 4;
  struct Group {
    typename PreLanes<T, CH>::type pp[kG];
    float dv[kG][CH], hp[kG][CH], xn[kG][CH];
  };
  auto load_group = [&](Group &G, int t0) {
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      const int t = t0 - u;
      if (t >= s) {
        const size_t o = base + static_cast<size_t>(t) * D;
        G.pp[u] = PreLanes<T, CH>::load(pre, o);
        Lanes<T, CH>::load(dy, o, G.dv[u]);
        if (t > 0) {
          Lanes<T, CH>::load(y, o - D, G.hp[u]);
        } else {
#pragma unroll
          for (int k = 0; k < CH; ++k) G.hp[u][k] = hinit[k];
        }
        if (t >= 4) {
          Lanes<T, CH>::load(x, o - 4 * static_cast<size_t>(D), G.xn[u]);
        } else {
#pragma unroll
          for (int k = 0; k < CH; ++k) G.xn[u][k] = 0.0f;
        }
      }
    }
  };
  auto run_group = [&](const Group &G, int t0) {
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      const int t = t0 - u;
      if (t >= s) {
        float dpa[CH], dpx[CH], dd[CH];
#pragma unroll
        for (int k = 0; k < CH; ++k) {
          const float xc =
              fmaf(w[3][k], xw[3][k], fmaf(w[2][k], xw[2][k], fmaf(w[1][k], xw[1][k], w[0][k] * xw[0][k])));
          const float r = fast_sigmoid(PrePair<T>::pa(G.pp[u].v[k]));
          const float ig = fast_sigmoid(PrePair<T>::px(G.pp[u].v[k]));
          const float em = expm1_nonpos(kd[k] * r);
          const float a = 1.0f + em;
          const float m = __builtin_amdgcn_sqrtf(-em * (2.0f + em));
          const float delta = G.dv[u][k] + g[k];
          const float dm = delta * ig * xc;
          const float di = delta * m * xc;
          float dz = delta * G.hp[u][k] * a;
          if (m > 0.0f) dz -= dm * (a * a) * __builtin_amdgcn_rcpf(m);
          dpa[k] = kd[k] * dz * (r * (1.0f - r));
          dpx[k] = di * (ig * (1.0f - ig));
          dd[k] = delta * m * ig;
          s_pa[k] += dpa[k];
          s_px[k] += dpx[k];
          s_rdz[k] = fmaf(r, dz, s_rdz[k]);
          g[k] = a * delta;
          xw[3][k] = xw[2][k];
          xw[2][k] = xw[1][k];
          xw[1][k] = xw[0][k];
          xw[0][k] = G.xn[u][k];
        }
        const size_t o = base + static_cast<size_t>(t) * D;
        DPair<T>::template put<CH>(dpre, o, dpa, dpx);
        DxcS<T, CH>::store(dxc, o, dd);
      }
    }
  };
  Group ga, gb;
  load_group(ga, e - 1);
  for (int t0 = e - 1; t0 >= s; t0 -= 2 * kG) {
    if (t0 - kG >= s) load_group(gb, t0 - kG);
    run_group(ga, t0);
    if (t0 - kG < s) break;
    if (t0 - 2 * kG >= s) load_group(ga, t0 - 2 * kG);
    run_group(gb, t0 - kG);
  }
  const size_t P = static_cast<size_t>(B) * nC * D;
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    part[cidx + k] = s_pa[k];
    part[P + cidx + k] = s_px[k];
    part[2 * P + cidx + k] = s_rdz[k];
  }
}

// ---- 4a: dxc += [dpa dpx] [W_a ; W_x] on MFMA (bf16 I/O, Dh in {32, 64, 128, 256}) ----------
// wti[g][i][2o + q] = W_q[g][o][i] (q = 0: W_a, 1: W_x) as fp16: the weights transposed and
// interleaved so that the contraction index k = 2o + q matches the (dpa, dpx) fp16 pair layout of
// dpre (fp16 holds every bf16 weight of magnitude 2^-14 .. 65504 exactly).
// One workgroup per (head, 32 o, 32 i) tile (Dh a multiple of 32): both gates' 32 x 32 blocks
// read as 16-byte row pieces into LDS (fp16), written out as 16-byte pieces of 32 wti rows.
__global__ __launch_bounds__(256) void wt_prep(const bf16_t *__restrict__ W_a,
                                               const bf16_t *__restrict__ W_x,
                                               uint16_t *__restrict__ wti, int H, int Dh) {
  __shared__ uint16_t tl[2][32][34];  // [gate][o][i] fp16 (rows padded)
  const int g = blockIdx.z, o0 = blockIdx.y * 32, i0 = blockIdx.x * 32;
  const int tid = threadIdx.x;
  {
    const int q = tid >> 7, r = (tid >> 2) & 31, c = tid & 3;
    const bf16_t *W = q ? W_x : W_a;
    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(
        W + (static_cast<size_t>(g) * Dh + o0 + r) * Dh + i0 + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t hv = pack_f16x2(bf16lo(v[e]), bf16hi(v[e]));
      tl[q][r][8 * c + 2 * e] = static_cast<uint16_t>(hv);
      tl[q][r][8 * c + 2 * e + 1] = static_cast<uint16_t>(hv >> 16);
    }
  }
  __syncthreads();
  {
    const int i = tid >> 3, c = tid & 7;  // row i0 + i; k = 2 o0 + 8 c ..: o = 4 c .. 4 c + 3
    u32x4_t out;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      out[m] = static_cast<uint32_t>(tl[0][4 * c + m][i]) |
               (static_cast<uint32_t>(tl[1][4 * c + m][i]) << 16);
    *reinterpret_cast<u32x4_t *>(wti + (static_cast<size_t>(g) * Dh + i0 + i) * 2 * Dh +
                                 2 * o0 + 8 * c) = out;
  }
}

template <int DH>
__global__ __launch_bounds__(kThreads) void dxc_mfma(const uint32_t *__restrict__ dpre,
                                                     const uint16_t *__restrict__ wti,
                                                     uint16_t *__restrict__ dxc, int Tn, int D) {
  typedef GateTile<DH> C;
  constexpr int K = 2 * DH;
  constexpr int kLd = K + 8;  // LDS row stride in fp16 (16 B pad)
  __shared__ __attribute__((aligned(16))) uint16_t lds_a[kTileRows * kLd];
  const int t0 = blockIdx.x * kTileRows;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  // A tile: rows t0..t0+63 of this head's K = 2 DH fp16 (DH pairs), zero past T.
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
  const uint16_t *wg = wti + static_cast<size_t>(g) * DH * K;
  f32x16_t acc[C::kGPW][C::kRPW];
#pragma unroll
  for (int gi = 0; gi < C::kGPW; ++gi)
#pragma unroll
    for (int ri = 0; ri < C::kRPW; ++ri) acc[gi][ri] = f32x16_t{};
#pragma unroll 2
  for (int k0 = 0; k0 < K; k0 += 16) {
    f16x8_t af[C::kRPW], bfr[C::kGPW];
#pragma unroll
    for (int ri = 0; ri < C::kRPW; ++ri)
      af[ri] = load_f16x8(lds_a + ((r0 + ri) * 32 + lrow) * kLd + k0 + khalf);
#pragma unroll
    for (int gi = 0; gi < C::kGPW; ++gi)
      bfr[gi] = load_f16x8(wg + static_cast<size_t>((g0 + gi) * 32 + lrow) * K + k0 + khalf);
#pragma unroll
    for (int gi = 0; gi < C::kGPW; ++gi)
#pragma unroll
      for (int ri = 0; ri < C::kRPW; ++ri)
        acc[gi][ri] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ri], bfr[gi], acc[gi][ri], 0, 0, 0);
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
          const size_t o = (static_cast<size_t>(b) * Tn + t) * D + d;
          DxcS<bf16_t>::st(dxc, o, DxcS<bf16_t>::ld(dxc, o) + acc[gi][ri][j]);
        }
      }
  }
}

// ---- 4b: the same on the vector ALU (fp32, or bf16 with other head sizes) -------------------
constexpr int kBwdValuRows = 16;

template <typename T>
__global__ __launch_bounds__(256) void dxc_valu(const typename DPair<T>::type *__restrict__ dpre,
                                                const T *__restrict__ W_a,
                                                const T *__restrict__ W_x,
                                                typename DxcS<T>::type *__restrict__ dxc,
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
      DPair<T>::get(dpre,
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
    const size_t o = (static_cast<size_t>(b) * Tn + t) * D + static_cast<size_t>(g) * Dh + i;
    DxcS<T>::st(dxc, o, DxcS<T>::ld(dxc, o) + acc);
  }
}

// ---- 5: conv backward -----------------------------------------------------------------------
// pcw: [B * nC][4][D] partial sums of dconv_w over each chunk.
template <typename T, int CH>
__global__ __launch_bounds__(kBwdThreads) void conv_bwd(const T *__restrict__ x,
                                                        const typename DxcS<T>::type *__restrict__ dxc,
                                                        const T *__restrict__ conv_w,
                                                        T *__restrict__ dx,
                                                        float *__restrict__ pcw, int B, int Tn,
                                                        int D, int nC) {
  const int DL = D / CH;
  const size_t idx = static_cast<size_t>(blockIdx.x) * kBwdThreads + threadIdx.x;
  if (idx >= static_cast<size_t>(B) * DL) return;
  const int b = static_cast<int>(idx / DL);
  const int d0 = static_cast<int>(idx % DL) * CH;
  const int c = blockIdx.y;
  const int s = c * kBwdChunk;
  const int e = min(s + kBwdChunk, Tn);
  float w[4][CH];
#pragma unroll
  for (int j = 0; j < 4; ++j) Lanes<T, CH>::load(conv_w, static_cast<size_t>(j) * D + d0, w[j]);
  const size_t base = static_cast<size_t>(b) * Tn * D + d0;
  // gw[k] = dxc[t + k] (zero at or past T); xw[j] = x[t - 3 + j] (zero before 0)
  float gw[4][CH], xw[4][CH];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    if (s + k < Tn) {
      DxcS<T, CH>::load(dxc, base + static_cast<size_t>(s + k) * D, gw[k + 1]);
    } else {
#pragma unroll
      for (int q = 0; q < CH; ++q) gw[k + 1][q] = 0.0f;
    }
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int q = s - 3 + j;
    if (q >= 0) {
      Lanes<T, CH>::load(x, base + static_cast<size_t>(q) * D, xw[j + 1]);
    } else {
#pragma unroll
      for (int k = 0; k < CH; ++k) xw[j + 1][k] = 0.0f;
    }
  }
  float acc[4][CH] = {};
  // groups of kG steps, double buffered (loads of group i+1 ahead of group i's stores)
  constexpr int kG = 4;
  struct Group {
    float gn[kG][CH], xn[kG][CH];
  };
  auto load_group = [&](Group &G, int t0) {
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      const int t = t0 + u;
      if (t < e) {
        if (t + 3 < Tn) {
          DxcS<T, CH>::load(dxc, base + static_cast<size_t>(t + 3) * D, G.gn[u]);
        } else {
#pragma unroll
          for (int k = 0; k < CH; ++k) G.gn[u][k] = 0.0f;
        }
        Lanes<T, CH>::load(x, base + static_cast<size_t>(t) * D, G.xn[u]);
      }
    }
  };
  auto run_group = [&](const Group &G, int t0) {
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      const int t = t0 + u;
      if (t < e) {
        float v[CH];
#pragma unroll
        for (int k = 0; k < CH; ++k) {
          gw[0][k] = gw[1][k];
          gw[1][k] = gw[2][k];
          gw[2][k] = gw[3][k];
          gw[3][k] = G.gn[u][k];
          xw[0][k] = xw[1][k];
          xw[1][k] = xw[2][k];
          xw[2][k] = xw[3][k];
          xw[3][k] = G.xn[u][k];
          // dx[t] = sum_j w[j] dxc[t + 3 - j]
          v[k] = fmaf(w[0][k], gw[3][k], fmaf(w[1][k], gw[2][k], fmaf(w[2][k], gw[1][k], w[3][k] * gw[0][k])));
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j][k] = fmaf(gw[0][k], xw[j][k], acc[j][k]);
        }
        Lanes<T, CH>::store(dx, base + static_cast<size_t>(t) * D, v);
      }
    }
  };
  Group ga, gb;
  load_group(ga, s);
  for (int t0 = s; t0 < e; t0 += 2 * kG) {
    if (t0 + kG < e) load_group(gb, t0 + kG);
    run_group(ga, t0);
    if (t0 + kG >= e) break;
    if (t0 + 2 * kG < e) load_group(ga, t0 + 2 * kG);
    run_group(gb, t0 + kG);
  }
  const size_t prow = (static_cast<size_t>(b) * nC + c) * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int k = 0; k < CH; ++k) pcw[(prow + j) * D + d0 + k] = acc[j][k];
}

// ---- 6a: dW partials on MFMA (bf16 I/O, Dh in {128, 256}) ----------------------------------
// One workgroup: a 256 (m = 2o + q, both gates interleaved) x Dh (i) tile of head g, contracted
// over the rows [kb, ke) of the flattened (b, t) index in steps of 32 rows; 8 waves (two per
// SIMD) in a 4 x 2 grid, each 64 x Dh/2 (2 x Dh/64 MFMA tiles, fp32 accumulators). Per step, dp
// and the conv output xc (recomputed from x in fp32) are written to LDS transposed, k
// contiguous, as pairs of rows: a row of 32 k plus 4 pad is 72 bytes, so the 4-byte stores of
// one instruction (16 row pairs x 2 octets of m per half-wave) hit 32 distinct banks and the
// 16-byte operand reads, taken as two 8-byte halves, distinct banks too. The LDS holds two
// steps and the registers the loads of two more: step s+2's loads are issued before step s's
// MFMAs, and step s+1 (loaded a step earlier) is converted into the other buffer after them,
// one barrier per step. (With one step of look-ahead each step waited for the round trip of the
// loads it had just issued: 133 against 104 us per call at B8 T2048 D2560 H10.)
// Precision: both operands in fp16 (dp as stored, xc rounded once), one MFMA per tile and k-step.
// With bf16 operands (2^-9) a dW element erred by up to a few percent of the tensor's rms -- dW
// sums terms of both signs and the gate gradients are heavy tailed (dz carries 1/m); fp16's 2^-11
// brings that well inside the bound, at a third of the matrix work of a hi + lo split.
// pw: [S][2 gates][H][Dh][Dh] fp32.
constexpr int kDwRows = 32;            // rows per step
constexpr int kDwLd = kDwRows + 4;     // LDS row stride in 16-bit words (72 bytes)
constexpr int kDwM = 256;              // m per workgroup
constexpr int kDwThreads = 512;

template <int DH> struct DwTile {
  static_assert(DH == 128 || DH == 256, "dW MFMA tile needs Dh in {128, 256}");
  static constexpr int kMt = 2 * DH / kDwM;        // m tiles per head
  static constexpr int kWN = DH / 64;              // 32-column MFMA tiles per wave
  static constexpr int kAElems = kDwM * kDwLd;     // [m][k]
  static constexpr int kBElems = DH * kDwLd;       // [i][k]
  static constexpr int kBufElems = kAElems + kBElems;
};

__device__ __forceinline__ f16x8_t lds_read_f16x8(const uint16_t *p) {
  const uint2 lo = *reinterpret_cast<const uint2 *>(p);
  const uint2 hi = *reinterpret_cast<const uint2 *>(p + 4);
  const u32x4_t v = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(f16x8_t, v);
}

template <int DH>
__global__ __launch_bounds__(kDwThreads, 1) void dw_mfma(const bf16_t *__restrict__ x,
                                                         const uint32_t *__restrict__ dpre,
                                                         const bf16_t *__restrict__ conv_w,
                                                         float *__restrict__ pw, int Tn, int D,
                                                         int H, int rows, int rows_per_split) {
  typedef DwTile<DH> C;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * C::kBufElems];
  // (head, split) groups in a 1-D grid. With two m tiles per head, the pair of workgroups that
  // share a group's x rows are 8 apart: workgroups go to the 8 XCDs round-robin, so both land
  // on one XCD and its L2 serves the second read of x.
  const int nsplit = (rows + rows_per_split - 1) / rows_per_split;
  int mt, grp;
  if constexpr (C::kMt == 1) {
    mt = 0;
    grp = blockIdx.x;
  } else {
    mt = (blockIdx.x >> 3) & 1;
    grp = (blockIdx.x >> 4) * 8 + (blockIdx.x & 7);
  }
  if (grp >= H * nsplit) return;  // padding of the last set of 16 (uniform per workgroup)
  const int g = grp % H;
  const int sp = grp / H;
  const int kb = sp * rows_per_split;
  const int ke = min(kb + rows_per_split, rows);
  const int nsteps = (ke - kb + kDwRows - 1) / kDwRows;
  const int tid = threadIdx.x;
  // loader roles: rows 2 lq, 2 lq + 1 of the step; A: 4 pairs (8 m) at octet lj; B: 8 channels
  // at octet lj (only lj < DH / 8 load B)
  const int lq = tid & 15;
  const int lj = tid >> 4;
  const bool bload = lj < DH / 8;
  const size_t a_col = static_cast<size_t>(g) * DH + (mt * kDwM + 8 * lj) / 2;  // uint32 pairs
  const int ich = 8 * (bload ? lj : 0);                                       // B channels
  const size_t b_col = static_cast<size_t>(g) * DH + ich;
  // conv taps of this thread's 8 channels as bf16 pairs (w0, w1) and (w2, w3): the conv output
  // is two bf16 dot products per channel with fp32 accumulation (the products are exact)
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  constexpr uint32_t kLoPair = 0x05040100u, kHiPair = 0x07060302u;  // low / high halves
  bf16x2_t w01[8], w23[8];
  {
    u32x4_t cwv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      cwv[j] = *reinterpret_cast<const u32x4_t *>(conv_w + static_cast<size_t>(j) * D + b_col);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      w01[2 * h] = __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(cwv[1][h], cwv[0][h], kLoPair));
      w01[2 * h + 1] = __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(cwv[1][h], cwv[0][h], kHiPair));
      w23[2 * h] = __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(cwv[3][h], cwv[2][h], kLoPair));
      w23[2 * h + 1] = __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(cwv[3][h], cwv[2][h], kHiPair));
    }
  }
  // prefetch registers: the dp rows [u] and x rows r0 - 3 .. r0 + 1 of a step; two sets, so
  // that a step's loads are in flight for two steps' MFMAs
  u32x4_t ra0[2], ra1[2];
  u32x4_t rx0[5], rx1[5];
  // The loads are unconditional, their rows clamped into the tensor (a load under a per-lane
  // branch makes the compiler wait for every outstanding load before the next use of any); rows
  // past the split are zeroed when the step is converted, and taps before a sequence's start by
  // the conv's own mask.
  auto load_step = [&](int st, u32x4_t (&pa)[2], u32x4_t (&rx)[5]) {
    const int r0 = kb + st * kDwRows + 2 * lq;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      pa[u] = *reinterpret_cast<const u32x4_t *>(
          dpre + static_cast<size_t>(min(r0 + u, rows - 1)) * D + a_col);
#pragma unroll
    for (int k = 0; k < 5; ++k)
      rx[k] = *reinterpret_cast<const u32x4_t *>(
          x + static_cast<size_t>(min(max(r0 - 3 + k, 0), rows - 1)) * D + b_col);
  };
  // conv, fp16 rounding and transposed stores of one step into buffer `buf`
  auto store_step = [&](int st, int buf, const u32x4_t (&pa)[2], const u32x4_t (&rx)[5]) {
    uint16_t *A = lds + buf * C::kBufElems;
    uint16_t *Bm = A + C::kAElems;
    const int k0 = kb + st * kDwRows;
    const int r0 = k0 + 2 * lq;
    const bool in0 = r0 < ke, in1 = r0 + 1 < ke;  // rows of this split
    // A: m = 8 lj + cc is half cc & 1 (dpa even, dpx odd) of pair cc >> 1; rows 2 lq, 2 lq + 1
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      *reinterpret_cast<uint32_t *>(A + (8 * lj + cc) * kDwLd + 2 * lq) = __builtin_amdgcn_perm(
          in1 ? pa[1][cc >> 1] : 0u, in0 ? pa[0][cc >> 1] : 0u, (cc & 1) ? kHiPair : kLoPair);
    // (every thread converts x rows at Dh 256; a per-lane branch here would cost the steady
    // loop its load accounting, as above)
    if (DH < 256 && !bload) return;
    // Does this step hold one of the first three rows of a sequence (uniform over the
    // workgroup)? Only then do conv taps need masking at the sequence start.
    const int f = k0 % Tn;
    const bool edge = f <= 2 || Tn - f <= kDwRows - 1 + 2;
    // tap j of output row u reads loaded row u + j; at a sequence start the taps before time 0
    // read zero instead (the rows loaded there belong to the previous sequence)
    const int t0 = r0 % Tn;
    float xcv[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // time of row r0 + u within its sequence (it wraps at most once: u <= 1)
      int t = t0 + u;
      if (t >= Tn) t -= Tn;
      uint32_t xw[4][4];  // [tap][word]
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = !edge || t - 3 + j >= 0;
#pragma unroll
        for (int h = 0; h < 4; ++h) xw[j][h] = ok ? rx[u + j][h] : 0u;
      }
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const uint32_t sel = (cc & 1) ? kHiPair : kLoPair;
        const int h = cc >> 1;
        const bf16x2_t p01 = __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(xw[1][h], xw[0][h], sel));
        const bf16x2_t p23 = __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(xw[3][h], xw[2][h], sel));
        xcv[u][cc] = __builtin_amdgcn_fdot2_f32_bf16(
            p23, w23[cc], __builtin_amdgcn_fdot2_f32_bf16(p01, w01[cc], 0.0f, false), false);
      }
    }
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      *reinterpret_cast<uint32_t *>(Bm + (8 * lj + cc) * kDwLd + 2 * lq) =
          pack_f16x2(in0 ? xcv[0][cc] : 0.0f, in1 ? xcv[1][cc] : 0.0f);
  };

  const int w = tid >> 6;
  const int lane = tid & 63;
  const int wm = (w & 3) * 64, wn = (w >> 2) * (DH / 2);
  const int lrow = lane & 31;
  const int khalf = (lane >> 5) * 8;
  f32x16_t acc[2][C::kWN];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < C::kWN; ++c) acc[a][c] = f32x16_t{};

  auto mfma_step = [&](int buf) {
    const uint16_t *A = lds + buf * C::kBufElems;
    const uint16_t *Bm = A + C::kAElems;
#pragma unroll
    for (int kk = 0; kk < kDwRows; kk += 16) {
      f16x8_t af[2];  // [m tile]
#pragma unroll
      for (int a = 0; a < 2; ++a)
        af[a] = lds_read_f16x8(A + (wm + a * 32 + lrow) * kDwLd + kk + khalf);
#pragma unroll
      for (int c = 0; c < C::kWN; ++c) {
        const f16x8_t bfr = lds_read_f16x8(Bm + (wn + c * 32 + lrow) * kDwLd + kk + khalf);
#pragma unroll
        for (int a = 0; a < 2; ++a)
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bfr, acc[a][c], 0, 0, 0);
      }
    }
  };
  // Step st: operands in LDS buffer st & 1. Its MFMAs run while step st + 1's loads (issued a
  // step earlier) and step st + 2's (issued now, into the registers step st's conversion has
  // freed) are in flight; step st + 1 is then converted into the other buffer. One step of
  // look-ahead left every step waiting on the round trip of the loads it had just issued.
  // The steady-state loop has no conditions: on a path that skips a step's loads the compiler
  // can no longer tell which loads are outstanding and waits for all of them. The last steps
  // (at most three) take the conditional form.
  auto body = [&](int st, const u32x4_t (&pa_next)[2], const u32x4_t (&rx_next)[5],
                  u32x4_t (&pa_free)[2], u32x4_t (&rx_free)[5]) {
    load_step(st + 2, pa_free, rx_free);
    __builtin_amdgcn_sched_barrier(0);  // the loads go out first, not after the conversion
    mfma_step(st & 1);
    store_step(st + 1, (st + 1) & 1, pa_next, rx_next);
    __syncthreads();
  };
  auto tail = [&](int st, const u32x4_t (&pa_next)[2], const u32x4_t (&rx_next)[5],
                  u32x4_t (&pa_free)[2], u32x4_t (&rx_free)[5]) {
    if (st >= nsteps) return;
    if (st + 2 < nsteps) load_step(st + 2, pa_free, rx_free);
    mfma_step(st & 1);
    if (st + 1 < nsteps) store_step(st + 1, (st + 1) & 1, pa_next, rx_next);
    __syncthreads();
  };
  load_step(0, ra0, rx0);
  if (nsteps > 1) load_step(1, ra1, rx1);
  store_step(0, 0, ra0, rx0);
  __syncthreads();
  int st = 0;
  for (; st + 3 < nsteps; st += 2) {
    body(st, ra1, rx1, ra0, rx0);
    body(st + 1, ra0, rx0, ra1, rx1);
  }
  tail(st, ra1, rx1, ra0, rx0);
  tail(st + 1, ra0, rx0, ra1, rx1);
  tail(st + 2, ra1, rx1, ra0, rx0);
  // ---- partial out: pw[sp][gate][g][o][i], m = 2 o + gate
  const size_t gstride = static_cast<size_t>(H) * DH * DH;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int m = mt * kDwM + wm + a * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
      float *dst = pw + (static_cast<size_t>(sp) * 2 + (m & 1)) * gstride +
                   (static_cast<size_t>(g) * DH + (m >> 1)) * DH + wn + lrow;
#pragma unroll
      for (int c = 0; c < C::kWN; ++c) dst[c * 32] = acc[a][c][j];
    }
}

// ---- 6b: dW partials on the vector ALU ------------------------------------------------------
// Output tile 64 (m) x 64 (i); 256 threads, each 4 x 4. Rows in steps of 16 staged in LDS.
template <typename T>
__global__ __launch_bounds__(256) void dw_valu(const T *__restrict__ x,
                                               const typename DPair<T>::type *__restrict__ dpre,
                                               const T *__restrict__ conv_w,
                                               float *__restrict__ pw, int Tn, int D, int H,
                                               int Dh, int rows, int rows_per_split) {
  __shared__ float sa[16][64], sb[16][64];
  const int nMt = (2 * Dh + 63) / 64;
  const int mt = blockIdx.x % nMt;
  const int nt = blockIdx.x / nMt;
  const int g = blockIdx.y;
  const int sp = blockIdx.z;
  const int kb = sp * rows_per_split;
  const int ke = min(kb + rows_per_split, rows);
  const int tid = threadIdx.x;
  const int tm = (tid & 15) * 4, tn = (tid >> 4) * 4;
  float acc[4][4] = {};
  for (int k0 = kb; k0 < ke; k0 += 16) {
    for (int q = tid; q < 16 * 64; q += 256) {
      const int r = q / 64, col = q % 64;
      const int rr = k0 + r;
      float va = 0.0f, vb = 0.0f;
      if (rr < ke) {
        const int bb = static_cast<int>(rr / Tn);
        const int t = static_cast<int>(rr % Tn);
        const size_t rowoff = (static_cast<size_t>(bb) * Tn + t) * D;
        const int m = mt * 64 + col;
        if (m < 2 * Dh) {
          float pa_, px_;
          DPair<T>::get(dpre, rowoff + static_cast<size_t>(g) * Dh + (m >> 1), pa_, px_);
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
  const size_t gstride = static_cast<size_t>(H) * Dh * Dh;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int m = mt * 64 + tm + u;
    if (m >= 2 * Dh) continue;
    float *dst = pw + (static_cast<size_t>(sp) * 2 + (m & 1)) * gstride +
                 (static_cast<size_t>(g) * Dh + (m >> 1)) * Dh;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = nt * 64 + tn + v;
      if (i < Dh) dst[i] = acc[u][v];
    }
  }
}

// ---- 7: fixed-order reduction of the partials ----------------------------------------------
// Segment y of the launch: out[j] = sum_{p < P} in[p ld + j] for j < n. A 256-thread block
// covers C = 256 / G columns with G interleaved partial sums each (p = q, q + G, ...), combined
// pairwise in a fixed tree -- a fixed order, so the result does not depend on scheduling. G is
// 16 for segments with many partials (the per-chunk vectors), 4 otherwise. With `lambda` set,
// out[j] is scaled by 8 sigmoid(-L_j) (dLambda from the sums of r dz).
// Segments with few partials over many columns (the dW splits) take G = 0 instead: each thread
// sums four adjacent columns (16-byte loads and store) over p = 0, 1, .. in order, with no tree
// (n, ld and both pointers then multiples of 4 floats; the host checks).
struct ColSum {
  const float *in;
  size_t ld, n;
  int P, G;
  float *out;
  const float *lambda;
};
constexpr int kMaxSeg = 6;
struct ColSums {
  ColSum seg[kMaxSeg];
};

__global__ __launch_bounds__(256) void colsum(ColSums segs) {
  __shared__ float red[256];
  const ColSum &sg = segs.seg[blockIdx.y];
  if (sg.G == 0) {
    const size_t j4 = (static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (j4 >= sg.n) return;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 4
    for (int p = 0; p < sg.P; ++p) {
      const float4 v = *reinterpret_cast<const float4 *>(sg.in + static_cast<size_t>(p) * sg.ld + j4);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    *reinterpret_cast<float4 *>(sg.out + j4) = acc;
    return;
  }
  const int G = sg.G, C = 256 / G;
  const int c = threadIdx.x % C, q = threadIdx.x / C;
  const size_t j = static_cast<size_t>(blockIdx.x) * C + c;
  if (static_cast<size_t>(blockIdx.x) * C >= sg.n) return;  // whole block past this segment
  float acc = 0.0f;
  if (j < sg.n) {
#pragma unroll 4
    for (int p = q; p < sg.P; p += G) acc += sg.in[static_cast<size_t>(p) * sg.ld + j];
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int h = G / 2; h > 0; h >>= 1) {  // fixed pairwise tree over the G partial sums
    if (q < h) red[threadIdx.x] += red[threadIdx.x + h * C];
    __syncthreads();
  }
  if (q == 0 && j < sg.n) {
    float v = red[c];
    if (sg.lambda) v *= kGateC / (1.0f + expf(sg.lambda[j]));
    sg.out[j] = v;
  }
}

// ---- host side ------------------------------------------------------------------------------
BwdLayout backward_layout(int B, int T, int D, int H, int io) {
  BwdLayout L;
  const int Dh = D / H;
  L.nC = (T + kBwdChunk - 1) / kBwdChunk;
  const long long rows = static_cast<long long>(B) * T;
  L.mfma_dxc = io == kBF16 && (Dh == 32 || Dh == 64 || Dh == 128 || Dh == 256);
  L.fused = io == kBF16 && static_cast<long long>(T) * D * 4 < (1LL << 31) &&
            fused_backward_supported(Dh);
  // partial sums of dpa, dpx, r dz: per chunk, or per tile of the fused pass
  L.nCp = L.fused ? (T + kFusedBwdRows - 1) / kFusedBwdRows : L.nC;
  L.mfma_dw = io == kBF16 && (Dh == 128 || Dh == 256);
  // Row splits of the dW contraction. MFMA: one 256 x Dh tile per workgroup and one workgroup
  // per CU (its LDS), so about as many workgroups as the 256 CUs of the chip, never more (a
  // second round would double the time). Vector ALU: about 1024 workgroups of 64 x 64 tiles.
  const long long tiles = L.mfma_dw ? static_cast<long long>(2 * Dh / kDwM) * H
                                    : static_cast<long long>((2 * Dh + 63) / 64) * ((Dh + 63) / 64) * H;
  const int step = L.mfma_dw ? kDwRows : 16;
  const long long steps = (rows + step - 1) / step;
  long long S = L.mfma_dw ? kBwdCUs / tiles : (1024 + tiles - 1) / tiles;
  S = std::max<long long>(1, std::min<long long>(S, std::min<long long>(steps, 65535)));
  L.rows_per_split = static_cast<int>((steps + S - 1) / S * step);
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
  // control words first, in every path: [1] counts look-back waits that gave up (read back by
  // rglru_lookback_failures), [2 + g] the tile tickets of the fused pass
  L.o_ctrl = take(kCtrlBytes);
  L.o_pre = take(L.fused ? 0 : n * pairb);
  L.o_dpre = take(n * pairb);
  L.o_dxc = take(n * (io == kBF16 ? 2 : 4));
  L.o_sums = take(L.fused ? 0 : P * D * sizeof(float2));
  L.o_carry = take(L.fused ? 0 : P * D * sizeof(float));
  L.o_part = take(3 * static_cast<size_t>(B) * L.nCp * D * sizeof(float));
  L.o_pcw = take(4 * P * D * sizeof(float));
  L.o_pw = take(static_cast<size_t>(L.S) * H * 2 * Dh * Dh * sizeof(float));
  L.o_wti = take(L.mfma_dxc ? static_cast<size_t>(H) * Dh * 2 * Dh * sizeof(bf16_t) : 0);
  L.o_lb = take(L.fused ? fused_backward_slots(B, T, D) * sizeof(unsigned long long) : 0);
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
  typename DxcS<T>::type *dxc = reinterpret_cast<typename DxcS<T>::type *>(ws + L.o_dxc);
  float2 *sums = reinterpret_cast<float2 *>(ws + L.o_sums);
  float *carry = reinterpret_cast<float *>(ws + L.o_carry);
  float *part = reinterpret_cast<float *>(ws + L.o_part);
  float *pcw = reinterpret_cast<float *>(ws + L.o_pcw);
  float *pw = reinterpret_cast<float *>(ws + L.o_pw);
  const bool resident = io == kBF16 && static_cast<long long>(Tn) * D * 4 < (1LL << 31);
  const size_t lanes = static_cast<size_t>(B) * D;
  const unsigned lblocks = static_cast<unsigned>((lanes + kBwdThreads - 1) / kBwdThreads);
  // lane kernels: two adjacent channels per lane when D is even
  const bool pair = D % 2 == 0;
  const dim3 lgrid(pair ? (lblocks + 1) / 2 : lblocks, L.nC);
  hipError_t e = hipSuccess;
  bool fused_conv = false;  // the dxc pass also ran the conv's transpose
  if (!L.fused) {
    // no waits on this path: the failure count is zero
    e = launch_clear_words(reinterpret_cast<unsigned *>(ws + L.o_ctrl), 2, s);
    if (e != hipSuccess) return e;
  }
  if constexpr (sizeof(T) == 2) {
    if (L.fused) {
      // passes 1-3 as one tile pass (partial sums per tile of kFusedBwdRows steps)
      e = launch_fused_backward(x, y, dy, h0, dh_T, conv_w, W_a, b_a, W_x, b_x, Lambda,
                                reinterpret_cast<uint32_t *>(dpre), dxc, part, dh0, B, Tn, D, H,
                                reinterpret_cast<unsigned *>(ws + L.o_ctrl),
                                reinterpret_cast<unsigned long long *>(ws + L.o_lb), s);
      if (e != hipSuccess) return e;
    }
  }
  if (!L.fused) {
    // pre-activations recomputed with the conv output split into bf16 hi + lo: the gradients
    // amplify pre-activation errors (through r (1 - r) and 1/m), so the backward does not reuse
    // the forward's bf16-operand rounding
    e = launch_gates(x, conv_w, W_a, b_a, W_x, b_x, pre, B, Tn, D, H, io, s, true);
    if (e != hipSuccess) return e;
    if (pair) {
      bwd_summary<T, 2><<<lgrid, kBwdThreads, 0, s>>>(pre, dy, Lambda, sums, B, Tn, D, L.nC);
    } else {
      bwd_summary<T, 1><<<lgrid, kBwdThreads, 0, s>>>(pre, dy, Lambda, sums, B, Tn, D, L.nC);
    }
    bwd_carry<<<lblocks, kBwdThreads, 0, s>>>(sums, dh_T, carry, dh0, B, D, L.nC);
    if (pair) {
      bwd_emit<T, 2><<<lgrid, kBwdThreads, 0, s>>>(x, pre, y, dy, h0, conv_w, Lambda, carry, dpre,
                                                   dxc, part, B, Tn, D, L.nC);
    } else {
      bwd_emit<T, 1><<<lgrid, kBwdThreads, 0, s>>>(x, pre, y, dy, h0, conv_w, Lambda, carry, dpre,
                                                   dxc, part, B, Tn, D, L.nC);
    }
  }
  if constexpr (sizeof(T) == 2) {
    if (L.mfma_dxc) {
      uint16_t *wti = reinterpret_cast<uint16_t *>(ws + L.o_wti);
      wt_prep<<<dim3(Dh / 32, Dh / 32, H), 256, 0, s>>>(W_a, W_x, wti, H, Dh);
      const dim3 grid((Tn + kTileRows - 1) / kTileRows, H, B);
      if (resident && resident_dxc_supported(Dh)) {
        // the conv's transpose included: dx and the dconv_w partials come out of this pass
        e = launch_resident_dxc(dpre, wti, dxc, x, conv_w, dx, pcw, B, Tn, D, H, s);
        if (e != hipSuccess) return e;
        fused_conv = true;
      } else switch (Dh) {
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
    dxc_valu<T><<<grid, 256, 0, s>>>(dpre, W_a, W_x, dxc, Tn, D, Dh);
  }
  // the conv backward reads and writes 16-bit values: four channels per lane (8-byte accesses)
  // where D allows it
  if (fused_conv) {
    // done by the dxc pass
  } else if (sizeof(T) == 2 && D % 4 == 0) {
    const dim3 qgrid((lblocks + 3) / 4, L.nC);
    if constexpr (sizeof(T) == 2)
      conv_bwd<T, 4><<<qgrid, kBwdThreads, 0, s>>>(x, dxc, conv_w, dx, pcw, B, Tn, D, L.nC);
  } else if (pair) {
    conv_bwd<T, 2><<<lgrid, kBwdThreads, 0, s>>>(x, dxc, conv_w, dx, pcw, B, Tn, D, L.nC);
  } else {
    conv_bwd<T, 1><<<lgrid, kBwdThreads, 0, s>>>(x, dxc, conv_w, dx, pcw, B, Tn, D, L.nC);
  }
  const int rows = B * Tn;  // < 2^31, checked by the caller
  if constexpr (sizeof(T) == 2) {
    if (L.mfma_dw) {
      // (head, split) groups; two m tiles per head at Dh 256 go out in sets of 16 workgroups
      const int groups = H * L.S;
      if (Dh == 256)
        dw_mfma<256><<<16 * ((groups + 7) / 8), kDwThreads, 0, s>>>(
            x, dpre, conv_w, pw, Tn, D, H, rows, L.rows_per_split);
      else
        dw_mfma<128><<<groups, kDwThreads, 0, s>>>(x, dpre, conv_w, pw, Tn, D, H, rows,
                                                    L.rows_per_split);
    }
  }
  if (!L.mfma_dw) {
    const dim3 grid(((2 * Dh + 63) / 64) * ((Dh + 63) / 64), H, L.S);
    dw_valu<T><<<grid, 256, 0, s>>>(x, dpre, conv_w, pw, Tn, D, H, Dh, rows,
                                     L.rows_per_split);
  }
  // fixed-order sums of the partials
  const int P = B * L.nC;
  const int Pp = B * L.nCp;  // partials of dpa, dpx, r dz
  const size_t PD = static_cast<size_t>(Pp) * D;
  const size_t nW = static_cast<size_t>(H) * Dh * Dh;
  ColSums cs;
  // 16 interleaved sums for the per-tile and per-chunk vectors (hundreds of partials over a few
  // thousand columns: with 4, their few blocks' serial load chains set the kernel's time; 32
  // and 64 measured slower again), 4 for the dW splits (about a dozen partials) when they cannot
  // take the four-column form
  const int GP = 16, GS = 4;
  cs.seg[0] = ColSum{part, static_cast<size_t>(D), static_cast<size_t>(D), Pp, GP, db_a, nullptr};
  cs.seg[1] = ColSum{part + PD, static_cast<size_t>(D), static_cast<size_t>(D), Pp, GP, db_x,
                     nullptr};
  cs.seg[2] = ColSum{part + 2 * PD, static_cast<size_t>(D), static_cast<size_t>(D), Pp, GP,
                     dLambda, Lambda};
  cs.seg[3] = ColSum{pcw, 4 * static_cast<size_t>(D), 4 * static_cast<size_t>(D), P, GP, dconv_w,
                     nullptr};
  // dW: four columns per thread where the layout allows 16-byte accesses
  auto al16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool v4 = nW % 4 == 0 && al16(pw) && al16(pw + nW) && al16(dW_a) && al16(dW_x);
  cs.seg[4] = ColSum{pw, 2 * nW, nW, L.S, v4 ? 0 : GS, dW_a, nullptr};
  cs.seg[5] = ColSum{pw + nW, 2 * nW, nW, L.S, v4 ? 0 : GS, dW_x, nullptr};
  size_t nblk = 0;
  for (int i = 0; i < kMaxSeg; ++i) {
    const size_t cols = cs.seg[i].G ? 256 / cs.seg[i].G : 1024;  // columns per block
    nblk = std::max(nblk, (cs.seg[i].n + cols - 1) / cols);
  }
  colsum<<<dim3(static_cast<unsigned>(nblk), kMaxSeg), 256, 0, s>>>(cs);
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
