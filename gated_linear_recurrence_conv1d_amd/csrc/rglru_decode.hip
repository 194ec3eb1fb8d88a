// rglru_decode.hip -- one batched, in-place decode step of the Conv1D -> RG-LRU block.
//
// The state has a fixed size whatever the sequence length (alby13 blog, "Core Components of
// Griffin -- 1. RG-LRU"; fast inference from it in "Griffin's Strengths"): per row, h[D] in fp32
// and the conv's last three inputs conv_state[3][D], oldest first. One step:
//   xc = w0 cs0 + w1 cs1 + w2 cs2 + w3 x_t;  gates from xc;  h <- a h + sqrt(1-a^2) i xc;
//   y_t = h;  conv_state <- (cs1, cs2, x_t).
// Every element of conv_state, h and y_t belongs to exactly one workgroup, which reads it before
// it writes it, so the in-place update needs no synchronisation beyond the workgroup's own.
//
//  * decode_mfma<DH>: bf16 I/O, DH in {32, 64}. A 32-row tile of one head: conv in fp32 into
//    LDS (fp32 copy for the gate math, bf16 copy as the MFMA A operand), the gate projections on
//    v_mfma_f32_32x32x16_bf16 with the weights streamed from L2 two k-steps ahead, then the
//    nonlinearity and state update straight from the accumulators. Every load that can be issued
//    early is (the states it updates, all conv-state rows of a thread), since a decode step is
//    one pass over memory with little compute to hide latency behind.
//  * decode_mfma64<DH>: bf16 I/O, DH in {128, 256}. The same on a 64-row tile, one wave per
//    32-channel group covering both 32-row halves, so each weight fragment streamed from L2 feeds
//    two MFMAs: the weights cross L2 once per 64 rows instead of per 32, which is what bounds the
//    MFMA phase (every workgroup streams its head's 2 Dh^2 weights at the same time).
//  * decode_valu<T>: any Dh <= 256, fp32 or bf16, one workgroup per (row, head).
#include "rglru_launch.h"
#include "rglru_mfma.h"

namespace rglru {

constexpr int kDecodeWord3 = 0x00020000;  // buffer descriptor word 3: raw 32-bit data, no swizzle

// Decode tile: 32 rows of one head, 4 waves. Wave w owns channel groups (32 channels each)
// w*kGPW .. w*kGPW+kGPW-1 for the 32 rows (waves past the last group only help with the conv).
// Small tiles give several workgroups per CU, whose load, compute and store phases overlap.
template <int DH> struct DecodeTile {
  static constexpr int kRows = 32;
  static constexpr int kGroups = DH / 32;
  static constexpr int kGPW = kGroups >= kWaves ? kGroups / kWaves : 1;
  static constexpr int kLda = DH + 8;  // LDS row stride in bf16 (16 B pad against conflicts)
  static constexpr int kKS = DH / 16;  // MFMA k-steps
  // Row of accumulator j in lane l (v_mfma_f32_32x32x16_bf16 layout).
  __device__ static int acc_row(int j, int lane) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); }
};

template <int DH>
__global__ __launch_bounds__(kThreads, 2) void decode_mfma(
    const bf16_t *__restrict__ x_t, bf16_t *__restrict__ cs, float *__restrict__ h,
    bf16_t *__restrict__ y_t, const bf16_t *__restrict__ conv_w, const bf16_t *__restrict__ W_a,
    const float *__restrict__ b_a, const bf16_t *__restrict__ W_x,
    const float *__restrict__ b_x, const float *__restrict__ Lambda, int N, int D) {
  typedef DecodeTile<DH> C;
  constexpr int kKS = C::kKS;
  __shared__ __attribute__((aligned(16))) bf16_t lds_a[C::kRows * C::kLda];
  __shared__ float lds_xc[C::kRows * DH];

  const int n0 = blockIdx.x * C::kRows;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int lrow = lane & 31;
  const int khalf = (lane >> 5) * 8;
  const int gq0 = w * C::kGPW;
  const bool active = gq0 < C::kGroups;

  // The fp32 states this wave will update are loaded first: they do not depend on the conv.
  float hv[C::kGPW][16];
  const size_t woff = static_cast<size_t>(g) * DH * DH;
  if (active) {
#pragma unroll
    for (int gi = 0; gi < C::kGPW; ++gi)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int n = min(n0 + C::acc_row(j, lane), N - 1);  // clamped; stores masked
        hv[gi][j] = h[static_cast<size_t>(n) * D + g * DH + (gq0 + gi) * 32 + lrow];
      }
  }

  // Conv and conv-state shift: thread = (channel pair p, rows r0 .. r0+RPG-1); all loads are
  // issued before any store (rows past N read row N-1 and store nothing).
  {
    constexpr int P = DH / 2;
    constexpr int RPG = C::kRows * P / kThreads;
    const int p = tid % P;
    const int r0 = (tid / P) * RPG;
    const int d0 = g * DH + 2 * p;
    float w0[4], w1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t wv = *reinterpret_cast<const uint32_t *>(conv_w + static_cast<size_t>(j) * D + d0);
      w0[j] = bf16lo(wv);
      w1[j] = bf16hi(wv);
    }
    uint32_t c0[RPG], c1[RPG], c2[RPG], xv[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const int n = min(n0 + r0 + i, N - 1);
      const uint32_t *c = reinterpret_cast<const uint32_t *>(cs + static_cast<size_t>(n) * 3 * D + d0);
      c0[i] = c[0];
      c1[i] = c[D / 2];
      c2[i] = c[D];
      xv[i] = *reinterpret_cast<const uint32_t *>(x_t + static_cast<size_t>(n) * D + d0);
    }
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const int r = r0 + i;
      const int n = n0 + r;
      const float y0 = fmaf(w0[3], bf16lo(xv[i]),
                            fmaf(w0[2], bf16lo(c2[i]), fmaf(w0[1], bf16lo(c1[i]), w0[0] * bf16lo(c0[i]))));
      const float y1 = fmaf(w1[3], bf16hi(xv[i]),
                            fmaf(w1[2], bf16hi(c2[i]), fmaf(w1[1], bf16hi(c1[i]), w1[0] * bf16hi(c0[i]))));
      if (n < N) {
        uint32_t *c = reinterpret_cast<uint32_t *>(cs + static_cast<size_t>(n) * 3 * D + d0);
        c[0] = c1[i];
        c[D / 2] = c2[i];
        c[D] = xv[i];
      }
      *reinterpret_cast<uint32_t *>(lds_a + r * C::kLda + 2 * p) = pack_bf16x2(y0, y1);
      lds_xc[r * DH + 2 * p] = y0;
      lds_xc[r * DH + 2 * p + 1] = y1;
    }
  }
  __syncthreads();
  if (!active) return;

  f32x16_t acc[C::kGPW][2];
#pragma unroll
  for (int gi = 0; gi < C::kGPW; ++gi) {
    acc[gi][0] = f32x16_t{};
    acc[gi][1] = f32x16_t{};
  }
  // weights from L2, two k-steps ahead of their MFMAs
  constexpr int kPF = 2;
  bf16x8_t bw[kPF][C::kGPW][2];
  auto load_w = [&](int ks, bf16x8_t (&dst)[C::kGPW][2]) {
#pragma unroll
    for (int gi = 0; gi < C::kGPW; ++gi) {
      const size_t wrow = woff + static_cast<size_t>((gq0 + gi) * 32 + lrow) * DH + ks * 16 + khalf;
      dst[gi][0] = load_bf16x8(W_a + wrow);
      dst[gi][1] = load_bf16x8(W_x + wrow);
    }
  };
#pragma unroll
  for (int i = 0; i < kPF && i < kKS; ++i) load_w(i, bw[i]);
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    const bf16x8_t af = load_bf16x8(lds_a + lrow * C::kLda + ks * 16 + khalf);
#pragma unroll
    for (int gi = 0; gi < C::kGPW; ++gi) {
      acc[gi][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bw[ks % kPF][gi][0], acc[gi][0], 0, 0, 0);
      acc[gi][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bw[ks % kPF][gi][1], acc[gi][1], 0, 0, 0);
    }
    if (ks + kPF < kKS) load_w(ks + kPF, bw[ks % kPF]);
  }

#pragma unroll
  for (int gi = 0; gi < C::kGPW; ++gi) {
    const int cl = (gq0 + gi) * 32 + lrow;
    const int d = g * DH + cl;
    const float ba = b_a[d], bx = b_x[d];
    const float kd = decay_coeff(Lambda[d]);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = C::acc_row(j, lane);
      const int n = n0 + row;
      if (n < N) {
        float a, u;
        gate(acc[gi][0][j] + ba, acc[gi][1][j] + bx, lds_xc[row * DH + cl], kd, a, u);
        const size_t off = static_cast<size_t>(n) * D + d;
        const float hn = fmaf(a, hv[gi][j], u);
        h[off] = hn;
        y_t[off] = f32_to_bf16(hn);
      }
    }
  }
}

// 64-row tile of one head: Dh/32 waves, wave w owns channel group w (32 channels) for rows
// 0..31 and 32..63 (accumulators [half][gate]); weights streamed from L2 kPF k-steps ahead.
template <int DH>
__global__ __launch_bounds__(2 * DH, 2) void decode_mfma64(
    const bf16_t *__restrict__ x_t, bf16_t *__restrict__ cs, float *__restrict__ h,
    bf16_t *__restrict__ y_t, const bf16_t *__restrict__ conv_w, const bf16_t *__restrict__ W_a,
    const float *__restrict__ b_a, const bf16_t *__restrict__ W_x,
    const float *__restrict__ b_x, const float *__restrict__ Lambda, int N, int D) {
  static_assert(DH == 128 || DH == 256, "64-row decode tile needs Dh in {128, 256}");
  constexpr int kRows = 64, kLda = DH + 8, kKS = DH / 16, kThr = 2 * DH, kPF = 4;
  __shared__ __attribute__((aligned(16))) bf16_t lds_a[kRows * kLda];
  __shared__ float lds_xc[kRows * DH];
  const int n0 = blockIdx.x * kRows;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int lrow = lane & 31;
  const int khalf = (lane >> 5) * 8;
  const int cl = w * 32 + lrow;  // this lane's channel within the head
  const int d = g * DH + cl;
  const float ba = b_a[d], bx = b_x[d];  // (loaded ahead of every store)
  const float kd = decay_coeff(Lambda[d]);
  // tile row of accumulator j in this lane (v_mfma_f32_32x32x16_bf16 layout), half 0
  auto acc_row = [&](int j) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); };

  // Every access goes through a buffer descriptor over its whole tensor (the launcher keeps
  // N * D * 6 bytes below 2^31): a row's byte offset is wave-uniform and a lane's fixed, so each
  // access costs one 32-bit add, and the range check reads zeros for rows past N and drops the
  // stores there (no clamps, no per-row branches; those rows only feed rows that are not stored).
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
      h, static_cast<short>(0), rec_bytes(N, D, 4u), kDecodeWord3);
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      cs, static_cast<short>(0), rec_bytes(N, 3 * D, 2u), kDecodeWord3);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(x_t), static_cast<short>(0), rec_bytes(N, D, 2u), kDecodeWord3);
  const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
      y_t, static_cast<short>(0), rec_bytes(N, D, 2u), kDecodeWord3);
  // this lane's element of accumulator row r of tile row block rb: element (n0 + rb + r) of
  // channel d, r = 8 (j >> 2) + (j & 3) wave-uniform, the half's 4-row shift in the lane offset
  const unsigned hl = static_cast<unsigned>(4 * (lane >> 5) * D + d);  // elements
  auto rowj = [&](int rt, int j) { return n0 + rt * 32 + 8 * (j >> 2) + (j & 3); };

  // The fp32 states this wave will update are loaded first: they do not depend on the conv.
  float hv[2][16];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      hv[rt][j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rh, static_cast<int>(row_bytes(rowj(rt, j), D, 4u) + 4u * hl), 0, 0));

  // Conv: thread = (channel pair p, rows r0 .. r0+RPG-1). The shifted conv state is stored only
  // after the MFMAs: vector memory operations complete in issue order, so stores issued here
  // would make every wait for a weight fragment in the MFMA loop wait for them as well.
  constexpr int P = DH / 2;
  constexpr int RPG = kRows * P / kThr;
  const int p = tid % P;
  const int r0 = (tid / P) * RPG;
  const int d0 = g * DH + 2 * p;
  uint32_t c1[RPG], c2[RPG], xv[RPG];
  {
    float w0[4], w1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t wv = *reinterpret_cast<const uint32_t *>(conv_w + static_cast<size_t>(j) * D + d0);
      w0[j] = bf16lo(wv);
      w1[j] = bf16hi(wv);
    }
    uint32_t c0[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const unsigned cb = row_bytes(n0 + r0 + i, 3 * D, 2u) + 2u * d0;
      c0[i] = __builtin_amdgcn_raw_buffer_load_b32(rc, static_cast<int>(cb), 0, 0);
      c1[i] = __builtin_amdgcn_raw_buffer_load_b32(rc, static_cast<int>(cb + 2u * D), 0, 0);
      c2[i] = __builtin_amdgcn_raw_buffer_load_b32(rc, static_cast<int>(cb + 4u * D), 0, 0);
      xv[i] = __builtin_amdgcn_raw_buffer_load_b32(
          rx, static_cast<int>(row_bytes(n0 + r0 + i, D, 2u) + 2u * d0), 0, 0);
    }
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const int r = r0 + i;
      const float y0 = fmaf(w0[3], bf16lo(xv[i]),
                            fmaf(w0[2], bf16lo(c2[i]), fmaf(w0[1], bf16lo(c1[i]), w0[0] * bf16lo(c0[i]))));
      const float y1 = fmaf(w1[3], bf16hi(xv[i]),
                            fmaf(w1[2], bf16hi(c2[i]), fmaf(w1[1], bf16hi(c1[i]), w1[0] * bf16hi(c0[i]))));
      *reinterpret_cast<uint32_t *>(lds_a + r * kLda + 2 * p) = pack_bf16x2(y0, y1);
      lds_xc[r * DH + 2 * p] = y0;
      lds_xc[r * DH + 2 * p + 1] = y1;
    }
  }
  __syncthreads();

  f32x16_t acc[2][2];  // [row half][gate]
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    acc[rt][0] = f32x16_t{};
    acc[rt][1] = f32x16_t{};
  }
  const size_t wrow = (static_cast<size_t>(g) * DH + cl) * DH + khalf;  // B operand: W row cl
  bf16x8_t bw[kPF][2];
#pragma unroll
  for (int i = 0; i < kPF && i < kKS; ++i) {
    bw[i][0] = load_bf16x8(W_a + wrow + i * 16);
    bw[i][1] = load_bf16x8(W_x + wrow + i * 16);
  }
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const bf16x8_t af = load_bf16x8(lds_a + (rt * 32 + lrow) * kLda + ks * 16 + khalf);
      acc[rt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bw[ks % kPF][0], acc[rt][0], 0, 0, 0);
      acc[rt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bw[ks % kPF][1], acc[rt][1], 0, 0, 0);
    }
    if (ks + kPF < kKS) {
      bw[ks % kPF][0] = load_bf16x8(W_a + wrow + (ks + kPF) * 16);
      bw[ks % kPF][1] = load_bf16x8(W_x + wrow + (ks + kPF) * 16);
    }
  }

  // conv-state shift (rows past N are dropped by the range check)
#pragma unroll
  for (int i = 0; i < RPG; ++i) {
    const unsigned cb = row_bytes(n0 + r0 + i, 3 * D, 2u) + 2u * d0;
    __builtin_amdgcn_raw_buffer_store_b32(c1[i], rc, static_cast<int>(cb), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(c2[i], rc, static_cast<int>(cb + 2u * D), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(xv[i], rc, static_cast<int>(cb + 4u * D), 0, 0);
  }
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = rt * 32 + acc_row(j);
      float a, u;
      gate(acc[rt][0][j] + ba, acc[rt][1][j] + bx, lds_xc[row * DH + cl], kd, a, u);
      const float hn = fmaf(a, hv[rt][j], u);
      __builtin_amdgcn_raw_buffer_store_b32(
          __float_as_uint(hn), rh, static_cast<int>(row_bytes(rowj(rt, j), D, 4u) + 4u * hl), 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16(
          __builtin_bit_cast(uint16_t, f32_to_bf16(hn)), ry,
          static_cast<int>(row_bytes(rowj(rt, j), D, 2u) + 2u * hl), 0, 0);
    }
}

template <typename T>
__global__ __launch_bounds__(256) void decode_valu(
    const T *__restrict__ x_t, T *__restrict__ cs, float *__restrict__ h, T *__restrict__ y_t,
    const T *__restrict__ conv_w, const T *__restrict__ W_a, const float *__restrict__ b_a,
    const T *__restrict__ W_x, const float *__restrict__ b_x, const float *__restrict__ Lambda,
    int D, int Dh) {
  __shared__ float xc[256];
  const int n = blockIdx.x;
  const int g = blockIdx.y;
  const int o = threadIdx.x;
  const int d = g * Dh + o;
  T *c = cs + static_cast<size_t>(n) * 3 * D;
  float xv = 0.0f, c1 = 0.0f, c2 = 0.0f;
  if (o < Dh) {
    const float c0 = Elem<T>::load(c, d);
    c1 = Elem<T>::load(c, static_cast<size_t>(D) + d);
    c2 = Elem<T>::load(c, static_cast<size_t>(2) * D + d);
    xv = Elem<T>::load(x_t, static_cast<size_t>(n) * D + d);
    float acc = Elem<T>::load(conv_w, d) * c0;
    acc = fmaf(Elem<T>::load(conv_w, static_cast<size_t>(D) + d), c1, acc);
    acc = fmaf(Elem<T>::load(conv_w, static_cast<size_t>(2) * D + d), c2, acc);
    acc = fmaf(Elem<T>::load(conv_w, static_cast<size_t>(3) * D + d), xv, acc);
    xc[o] = acc;
  }
  __syncthreads();
  if (o >= Dh) return;
  // shift the conv state (values were read above; stores are exact copies of dtype values)
  Elem<T>::store(c, d, c1);
  Elem<T>::store(c, static_cast<size_t>(D) + d, c2);
  Elem<T>::store(c, static_cast<size_t>(2) * D + d, xv);
  const size_t wr = (static_cast<size_t>(g) * Dh + o) * Dh;
  float sa = 0.0f, sx = 0.0f;
  for (int i = 0; i < Dh; ++i) {
    sa = fmaf(Elem<T>::load(W_a, wr + i), xc[i], sa);
    sx = fmaf(Elem<T>::load(W_x, wr + i), xc[i], sx);
  }
  float a, u;
  gate(sa + b_a[d], sx + b_x[d], xc[o], decay_coeff(Lambda[d]), a, u);
  const size_t off = static_cast<size_t>(n) * D + d;
  const float hn = fmaf(a, h[off], u);
  h[off] = hn;
  Elem<T>::store(y_t, off, hn);
}

// Prefill -> decode hand-off: conv_state[b][j] = x[b][T - 3 + j] (oldest first), zero where
// T - 3 + j < 0 -- the conv's view of the inputs before the next step, exactly as the forward saw
// them (zero padding before t = 0). 16-byte pieces when D allows, else elements.
template <typename T, int V>
__global__ __launch_bounds__(256) void prefill_state(const T *__restrict__ x, T *__restrict__ cs,
                                                     int B, int Tn, int D) {
  const int DV = D / V;
  const size_t n = static_cast<size_t>(B) * 3 * DV;
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int dv = static_cast<int>(i % DV);
  const size_t bj = i / DV;
  const int j = static_cast<int>(bj % 3);
  const int b = static_cast<int>(bj / 3);
  const int t = Tn - 3 + j;
  typedef u32x4_t P;
  const size_t dst = (bj * D + static_cast<size_t>(dv) * V);
  if constexpr (V * sizeof(T) == 16) {
    P v = {0u, 0u, 0u, 0u};
    if (t >= 0) v = *reinterpret_cast<const P *>(x + (static_cast<size_t>(b) * Tn + t) * D + dv * V);
    *reinterpret_cast<P *>(cs + dst) = v;
  } else {
    cs[dst] = t >= 0 ? x[(static_cast<size_t>(b) * Tn + t) * D + dv] : T(0);
  }
}

hipError_t launch_prefill_state(const void *x, void *conv_state, int B, int T, int D, int io,
                                hipStream_t s) {
  const size_t eb = io == kBF16 ? 2 : 4;
  const bool vec = (D * eb) % 16 == 0;
  const int V = vec ? static_cast<int>(16 / eb) : 1;
  const size_t n = static_cast<size_t>(B) * 3 * (D / V);
  const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
  if (io == kBF16) {
    if (vec)
      prefill_state<bf16_t, 8><<<blocks, 256, 0, s>>>(static_cast<const bf16_t *>(x),
                                                       static_cast<bf16_t *>(conv_state), B, T, D);
    else
      prefill_state<bf16_t, 1><<<blocks, 256, 0, s>>>(static_cast<const bf16_t *>(x),
                                                       static_cast<bf16_t *>(conv_state), B, T, D);
  } else {
    if (vec)
      prefill_state<float, 4><<<blocks, 256, 0, s>>>(static_cast<const float *>(x),
                                                     static_cast<float *>(conv_state), B, T, D);
    else
      prefill_state<float, 1><<<blocks, 256, 0, s>>>(static_cast<const float *>(x),
                                                     static_cast<float *>(conv_state), B, T, D);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const void *x_t, void *conv_state, float *h, void *y_t,
                         const void *conv_w, const void *W_a, const float *b_a, const void *W_x,
                         const float *b_x, const float *Lambda, int N, int D, int H, int io,
                         hipStream_t s) {
  const int Dh = D / H;
  // decode_mfma64 addresses its largest tensor (conv_state, 6 bytes per row and channel) with
  // 32-bit buffer offsets; larger batches take decode_valu
  const bool mfma64_fits = static_cast<long long>(N) * D * 6 < (1LL << 31);
  if (io == kBF16 && (Dh == 32 || Dh == 64 || ((Dh == 128 || Dh == 256) && mfma64_fits))) {
    dim3 grid((N + 31) / 32, H);    // DecodeTile<>::kRows rows per workgroup
    dim3 grid64((N + 63) / 64, H);  // decode_mfma64: 64 rows per workgroup
    const bf16_t *xx = static_cast<const bf16_t *>(x_t);
    bf16_t *cc = static_cast<bf16_t *>(conv_state);
    bf16_t *yy = static_cast<bf16_t *>(y_t);
    const bf16_t *cw = static_cast<const bf16_t *>(conv_w);
    const bf16_t *wa = static_cast<const bf16_t *>(W_a);
    const bf16_t *wx = static_cast<const bf16_t *>(W_x);
#define RGLRU_DECODE_CASE(DHV)                                                                  \
  case DHV:                                                                                     \
    decode_mfma<DHV><<<grid, kThreads, 0, s>>>(xx, cc, h, yy, cw, wa, b_a, wx, b_x, Lambda, N, \
                                               D);                                              \
    break;
    switch (Dh) {
      RGLRU_DECODE_CASE(32)
      RGLRU_DECODE_CASE(64)
      case 128:
        decode_mfma64<128><<<grid64, 256, 0, s>>>(xx, cc, h, yy, cw, wa, b_a, wx, b_x, Lambda, N, D);
        break;
      case 256:
        decode_mfma64<256><<<grid64, 512, 0, s>>>(xx, cc, h, yy, cw, wa, b_a, wx, b_x, Lambda, N, D);
        break;
      default: return hipErrorInvalidValue;
    }
#undef RGLRU_DECODE_CASE
    return hipGetLastError();
  }
  dim3 grid(N, H);
  if (io == kBF16) {
    decode_valu<bf16_t><<<grid, 256, 0, s>>>(
        static_cast<const bf16_t *>(x_t), static_cast<bf16_t *>(conv_state), h,
        static_cast<bf16_t *>(y_t), static_cast<const bf16_t *>(conv_w),
        static_cast<const bf16_t *>(W_a), b_a, static_cast<const bf16_t *>(W_x), b_x, Lambda, D,
        Dh);
  } else {
    decode_valu<float><<<grid, 256, 0, s>>>(
        static_cast<const float *>(x_t), static_cast<float *>(conv_state), h,
        static_cast<float *>(y_t), static_cast<const float *>(conv_w),
        static_cast<const float *>(W_a), b_a, static_cast<const float *>(W_x), b_x, Lambda, D,
        Dh);
  }
  return hipGetLastError();
}

}  // namespace rglru
