// rglru_gates.hip -- gate projections of the RG-LRU with the temporal Conv1D fused in front.
//
// pre[b][t][d] = (b_a[d] + (W_a[g] xc_t)[o], b_x[d] + (W_x[g] xc_t)[o]) with
// xc_t = causal depthwise conv of width 4 (Soham De's Griffin thread, tweet on keeping the
// recurrent block simple; the gates are state-free, alby13 blog, "Core Components of Griffin --
// 1. RG-LRU", which is what lets them run as one batched contraction ahead of the scan).
//
// bf16 I/O with Dh in {32, 64, 128, 256} goes to tile_preacts (rglru_bwd_tiles.hip: persistent
// workgroups, one head each, weights resident in registers) whenever one sequence fits 32-bit
// buffer offsets; otherwise to one of the kernels here:
//  * gates_mfma<DH>: bf16 I/O, DH in {32, 64, 128, 256}. Conv in fp32 into an LDS tile (rounded
//    to bf16 for the MFMA A operand), then the 64 x 2DH tile on v_mfma_f32_32x32x16_bf16 with
//    fp32 accumulation, the weights streamed from L2 per tile; fp16 (pa, px) pairs out.
//  * gates_tiled<T> (Dh % 4 == 0) and gates_valu<T> (any Dh <= 256): fp32 or bf16 I/O, plain
//    fp32 FMAs (used for fp32 I/O, where the 1e-4 accuracy target leaves no room for bf16
//    operands, and for other head sizes); the same sums in the same order, tiled or not.
#include "rglru_launch.h"
#include "rglru_mfma.h"

namespace rglru {

template <int DH, bool SPLIT>
__global__ __launch_bounds__(kThreads) void gates_mfma(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ conv_w,
    const bf16_t *__restrict__ W_a, const float *__restrict__ b_a,
    const bf16_t *__restrict__ W_x, const float *__restrict__ b_x, uint32_t *__restrict__ pre,
    int T, int D) {
  typedef GateTile<DH> C;
  // conv output rounded to bf16; with SPLIT also its residual, in the second half
  __shared__ __attribute__((aligned(16))) bf16_t lds_a[(SPLIT ? 2 : 1) * kTileRows * C::kLda];

  const int t0 = blockIdx.x * kTileRows;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;

  // ---- conv prologue: thread = (channel pair p, row group rg); sliding window over its rows.
  {
    constexpr int P = DH / 2;
    constexpr int RPG = kTileRows * P / kThreads;  // rows per thread
    const int p = tid % P;
    const int r0 = (tid / P) * RPG;
    const int d0 = g * DH + 2 * p;
    const uint32_t *xb = reinterpret_cast<const uint32_t *>(x + static_cast<size_t>(b) * T * D);
    float w0[4], w1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t wv = *reinterpret_cast<const uint32_t *>(conv_w + static_cast<size_t>(j) * D + d0);
      w0[j] = bf16lo(wv);
      w1[j] = bf16hi(wv);
    }
    float a0[3], a1[3];  // x[t-3], x[t-2], x[t-1] for the two channels
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      int t = t0 + r0 - 3 + k;
      uint32_t v = (t >= 0 && t < T) ? xb[(static_cast<size_t>(t) * D + d0) >> 1] : 0u;
      a0[k] = bf16lo(v);
      a1[k] = bf16hi(v);
    }
#pragma unroll 4
    for (int r = 0; r < RPG; ++r) {
      int t = t0 + r0 + r;
      uint32_t v = (t < T) ? xb[(static_cast<size_t>(t) * D + d0) >> 1] : 0u;
      float c0 = bf16lo(v), c1 = bf16hi(v);
      float y0 = fmaf(w0[3], c0, fmaf(w0[2], a0[2], fmaf(w0[1], a0[1], w0[0] * a0[0])));
      float y1 = fmaf(w1[3], c1, fmaf(w1[2], a1[2], fmaf(w1[1], a1[1], w1[0] * a1[0])));
      const uint32_t hi = pack_bf16x2(y0, y1);
      *reinterpret_cast<uint32_t *>(lds_a + (r0 + r) * C::kLda + 2 * p) = hi;
      if constexpr (SPLIT)
        *reinterpret_cast<uint32_t *>(lds_a + (kTileRows + r0 + r) * C::kLda + 2 * p) =
            pack_bf16x2(y0 - bf16lo(hi), y1 - bf16hi(hi));
      a0[0] = a0[1]; a0[1] = a0[2]; a0[2] = c0;
      a1[0] = a1[1]; a1[1] = a1[2]; a1[2] = c1;
    }
  }
  __syncthreads();

  const int w = tid >> 6;
  const int lane = tid & 63;
  int gq0, rq0;
  bool active;
  C::assign(w, gq0, rq0, active);
  if (!active) return;

  f32x16_t acc[C::kGPW][C::kRPW][2];
  const size_t woff = static_cast<size_t>(g) * DH * DH;
  gate_tile_mfma<DH, SPLIT>(lds_a, W_a + woff, W_x + woff, gq0, rq0, lane, acc,
                            lds_a + kTileRows * C::kLda);

  // ---- epilogue: bias, fp16 pair, store.
#pragma unroll
  for (int gi = 0; gi < C::kGPW; ++gi) {
    const int d = g * DH + (gq0 + gi) * 32 + (lane & 31);
    const float ba = b_a[d], bx = b_x[d];
#pragma unroll
    for (int ri = 0; ri < C::kRPW; ++ri)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int t = t0 + C::acc_row(rq0 + ri, j, lane);
        if (t < T)
          pre[(static_cast<size_t>(b) * T + t) * D + d] =
              pack_f16x2(acc[gi][ri][0][j] + ba, acc[gi][ri][1][j] + bx);
      }
  }
}

// ----------------------------------------------------------------------------------------------
constexpr int kValuRows = 16;

template <typename T>
__global__ __launch_bounds__(256) void gates_valu(
    const T *__restrict__ x, const T *__restrict__ conv_w, const T *__restrict__ W_a,
    const float *__restrict__ b_a, const T *__restrict__ W_x, const float *__restrict__ b_x,
    typename PrePair<T>::type *__restrict__ pre, int Tn, int D, int Dh) {
  __shared__ float xc[kValuRows * 256];
  const int t0 = blockIdx.x * kValuRows;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const T *xb = x + static_cast<size_t>(b) * Tn * D;
  for (int e = threadIdx.x; e < kValuRows * Dh; e += blockDim.x) {
    const int r = e / Dh, i = e % Dh;
    const int d = g * Dh + i;
    const int t = t0 + r;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < kConvW; ++j) {
      const int s = t - (kConvW - 1) + j;
      if (s >= 0 && s < Tn)
        acc = fmaf(Elem<T>::load(conv_w, static_cast<size_t>(j) * D + d),
                   Elem<T>::load(xb, static_cast<size_t>(s) * D + d), acc);
    }
    xc[r * Dh + i] = acc;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kValuRows * Dh; e += blockDim.x) {
    const int r = e / Dh, o = e % Dh;
    const int t = t0 + r;
    if (t >= Tn) continue;
    const int d = g * Dh + o;
    const size_t wr = (static_cast<size_t>(g) * Dh + o) * Dh;
    float sa = 0.0f, sx = 0.0f;
    for (int i = 0; i < Dh; ++i) {
      const float v = xc[r * Dh + i];
      sa = fmaf(Elem<T>::load(W_a, wr + i), v, sa);
      sx = fmaf(Elem<T>::load(W_x, wr + i), v, sx);
    }
    pre[(static_cast<size_t>(b) * Tn + t) * D + d] = PrePair<T>::pack(sa + b_a[d], sx + b_x[d]);
  }
}

// ----------------------------------------------------------------------------------------------
// gates_tiled<T>: the fp32-FMA contraction register-tiled, for Dh % 4 == 0 (Dh <= 256). A
// workgroup owns 64 rows of one head and 128 of its output channels: the conv output of the rows
// sits in LDS as fp32; wave w takes rows 16w .. 16w+15 and lane l the outputs l and l + 64, both
// gates, so each weight row is read by one lane as runs of 4 consecutive k (one 16-byte load for
// fp32; two such runs per chunk when Dh % 8 == 0), and each conv value is one LDS broadcast
// shared by the 64 lanes and reused for 4 FMAs.
// Every output is accumulated in ascending k from zero, as gates_valu does, so the two kernels
// agree bit for bit.
constexpr int kTiledRows = 64;
constexpr int kTiledOut = 128;
constexpr int kTiledK = 8;  // k per weight-row run (two 16-byte loads for fp32) when Dh allows

template <typename T> __device__ __forceinline__ float4 load4(const T *p);
template <> __device__ __forceinline__ float4 load4<float>(const float *p) {
  return *reinterpret_cast<const float4 *>(p);
}
template <> __device__ __forceinline__ float4 load4<bf16_t>(const bf16_t *p) {
  const uint2 v = *reinterpret_cast<const uint2 *>(p);
  return make_float4(bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y));
}

template <typename T, int KC>
__global__ __launch_bounds__(256) void gates_tiled(
    const T *__restrict__ x, const T *__restrict__ conv_w, const T *__restrict__ W_a,
    const float *__restrict__ b_a, const T *__restrict__ W_x, const float *__restrict__ b_x,
    typename PrePair<T>::type *__restrict__ pre, int Tn, int D, int Dh) {
  __shared__ float4 xc4[kTiledRows * 256 / 4];  // [row][Dh] fp32 conv output
  float *xc = reinterpret_cast<float *>(xc4);
  const int nob = (Dh + kTiledOut - 1) / kTiledOut;
  const int t0 = blockIdx.x * kTiledRows;
  const int g = blockIdx.y / nob;
  const int ob = blockIdx.y % nob;
  const int b = blockIdx.z;
  const T *xb = x + static_cast<size_t>(b) * Tn * D;
  for (int e = threadIdx.x; e < kTiledRows * Dh; e += blockDim.x) {
    const int r = e / Dh, i = e % Dh;
    const int d = g * Dh + i;
    const int t = t0 + r;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < kConvW; ++j) {
      const int s = t - (kConvW - 1) + j;
      if (s >= 0 && s < Tn)
        acc = fmaf(Elem<T>::load(conv_w, static_cast<size_t>(j) * D + d),
                   Elem<T>::load(xb, static_cast<size_t>(s) * D + d), acc);
    }
    xc[e] = acc;
  }
  __syncthreads();
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int o0 = ob * kTiledOut + lane;
  const int o1 = o0 + 64;
  // rows of out-of-range outputs are clamped to a valid one (loaded, never stored)
  const size_t wr0 = (static_cast<size_t>(g) * Dh + min(o0, Dh - 1)) * Dh;
  const size_t wr1 = (static_cast<size_t>(g) * Dh + min(o1, Dh - 1)) * Dh;
  const int rbase = w * 16;
  float acc[16][2][2];  // [row][output][gate]
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r][0][0] = acc[r][0][1] = acc[r][1][0] = acc[r][1][1] = 0.0f;
  constexpr int NV = KC / 4;  // runs of 4 k per weight row and chunk
  float4 wn[NV][4];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    wn[u][0] = load4<T>(W_a + wr0 + 4 * u);
    wn[u][1] = load4<T>(W_x + wr0 + 4 * u);
    wn[u][2] = load4<T>(W_a + wr1 + 4 * u);
    wn[u][3] = load4<T>(W_x + wr1 + 4 * u);
  }
  for (int k = 0; k < Dh; k += KC) {
    float4 wc[NV][4];
#pragma unroll
    for (int u = 0; u < NV; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) wc[u][c] = wn[u][c];
    if (k + KC < Dh) {
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        wn[u][0] = load4<T>(W_a + wr0 + k + KC + 4 * u);
        wn[u][1] = load4<T>(W_x + wr0 + k + KC + 4 * u);
        wn[u][2] = load4<T>(W_a + wr1 + k + KC + 4 * u);
        wn[u][3] = load4<T>(W_x + wr1 + k + KC + 4 * u);
      }
    }
#pragma unroll
    for (int u = 0; u < NV; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float4 v = xc4[((rbase + r) * Dh + k + 4 * u) >> 2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float4 a = wc[u][2 * q], xw = wc[u][2 * q + 1];
        acc[r][q][0] = fmaf(a.x, v.x, acc[r][q][0]);
        acc[r][q][1] = fmaf(xw.x, v.x, acc[r][q][1]);
        acc[r][q][0] = fmaf(a.y, v.y, acc[r][q][0]);
        acc[r][q][1] = fmaf(xw.y, v.y, acc[r][q][1]);
        acc[r][q][0] = fmaf(a.z, v.z, acc[r][q][0]);
        acc[r][q][1] = fmaf(xw.z, v.z, acc[r][q][1]);
        acc[r][q][0] = fmaf(a.w, v.w, acc[r][q][0]);
        acc[r][q][1] = fmaf(xw.w, v.w, acc[r][q][1]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int o = q ? o1 : o0;
    if (o >= Dh) continue;
    const int d = g * Dh + o;
    const float ba = b_a[d], bx = b_x[d];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + rbase + r;
      if (t < Tn)
        pre[(static_cast<size_t>(b) * Tn + t) * D + d] =
            PrePair<T>::pack(acc[r][q][0] + ba, acc[r][q][1] + bx);
    }
  }
}

// ----------------------------------------------------------------------------------------------
hipError_t launch_gates(const void *x, const void *conv_w, const void *W_a, const float *b_a,
                        const void *W_x, const float *b_x, void *pre, int B, int T, int D, int H,
                        int io, hipStream_t s, bool split) {
  const int Dh = D / H;
  if (io == kBF16 && resident_preacts_supported(Dh) &&
      static_cast<long long>(T) * D * 4 < (1LL << 31))
    return launch_resident_preacts(x, conv_w, W_a, b_a, W_x, b_x, pre, B, T, D, H, s, split);
  if (io == kBF16 && (Dh == 32 || Dh == 64 || Dh == 128 || Dh == 256)) {
    dim3 grid((T + kTileRows - 1) / kTileRows, H, B);
    const bf16_t *xx = static_cast<const bf16_t *>(x);
    const bf16_t *cw = static_cast<const bf16_t *>(conv_w);
    const bf16_t *wa = static_cast<const bf16_t *>(W_a);
    const bf16_t *wx = static_cast<const bf16_t *>(W_x);
    uint32_t *pp = static_cast<uint32_t *>(pre);
#define RGLRU_GATES_CASE(DHV)                                                                   \
  case DHV:                                                                                      \
    if (split)                                                                                   \
      gates_mfma<DHV, true><<<grid, kThreads, 0, s>>>(xx, cw, wa, b_a, wx, b_x, pp, T, D);       \
    else                                                                                         \
      gates_mfma<DHV, false><<<grid, kThreads, 0, s>>>(xx, cw, wa, b_a, wx, b_x, pp, T, D);      \
    break;
    switch (Dh) {
      RGLRU_GATES_CASE(32)
      RGLRU_GATES_CASE(64)
      RGLRU_GATES_CASE(128)
      RGLRU_GATES_CASE(256)
      default: return hipErrorInvalidValue;
    }
#undef RGLRU_GATES_CASE
    return hipGetLastError();
  }
  if (Dh % 4 == 0 && Dh <= 256 &&
      static_cast<long long>(H) * ((Dh + kTiledOut - 1) / kTiledOut) <= 65535) {
    dim3 tgrid((T + kTiledRows - 1) / kTiledRows, H * ((Dh + kTiledOut - 1) / kTiledOut), B);
#define RGLRU_TILED(TT, KCV, PT)                                                                  \
  gates_tiled<TT, KCV><<<tgrid, 256, 0, s>>>(                                                     \
      static_cast<const TT *>(x), static_cast<const TT *>(conv_w), static_cast<const TT *>(W_a),  \
      b_a, static_cast<const TT *>(W_x), b_x, static_cast<PT *>(pre), T, D, Dh)
    if (io == kBF16) {
      if (Dh % kTiledK == 0) RGLRU_TILED(bf16_t, kTiledK, uint32_t);
      else RGLRU_TILED(bf16_t, 4, uint32_t);
    } else {
      if (Dh % kTiledK == 0) RGLRU_TILED(float, kTiledK, float2);
      else RGLRU_TILED(float, 4, float2);
    }
#undef RGLRU_TILED
    return hipGetLastError();
  }
  dim3 grid((T + kValuRows - 1) / kValuRows, H, B);
  if (io == kBF16) {
    gates_valu<bf16_t><<<grid, 256, 0, s>>>(
        static_cast<const bf16_t *>(x), static_cast<const bf16_t *>(conv_w),
        static_cast<const bf16_t *>(W_a), b_a, static_cast<const bf16_t *>(W_x), b_x,
        static_cast<uint32_t *>(pre), T, D, Dh);
  } else {
    gates_valu<float><<<grid, 256, 0, s>>>(
        static_cast<const float *>(x), static_cast<const float *>(conv_w),
        static_cast<const float *>(W_a), b_a, static_cast<const float *>(W_x), b_x,
        static_cast<float2 *>(pre), T, D, Dh);
  }
  return hipGetLastError();
}

}  // namespace rglru
