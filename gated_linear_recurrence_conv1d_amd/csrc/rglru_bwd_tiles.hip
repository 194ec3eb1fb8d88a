// rglru_bwd_tiles.hip -- the two weight contractions of the backward pass as persistent
// workgroups with the weights resident in registers (bf16 I/O).
//
//  * tile_preacts<DH>: the gate pre-activations (pa, px) of every (b, t) row, recomputed from x:
//    causal conv of width 4 (Soham De's Griffin thread, tweet on keeping the recurrent block
//    simple), then [64 rows x Dh] x [Dh x 2Dh] per tile on MFMA (the gates do not read the
//    state, alby13 blog, "Core Components of Griffin -- 1. RG-LRU"). The conv output enters the
//    contraction as bf16 hi + lo (two MFMAs against the exact bf16 weights), because the
//    gradients amplify pre-activation errors through r (1 - r) and 1/m.
//  * tile_dxc<DH>: dxc += [dpa dpx] [W_a ; W_x], the gradient that flows back through the gate
//    projections into the conv output: [64 rows x 2Dh] x [2Dh x Dh] per tile.
//
// Both: one workgroup owns one head for its whole life and takes that head's 64-row tiles
// (time-major within a sequence, sequences in turn) in a static round robin; wave w owns the
// head's output channels in groups of 32 (two groups per wave at Dh = 256, one wave per SIMD)
// and keeps their weight rows -- the MFMA B operand, 256 registers at Dh = 256 -- in registers.
// The rows of tile k+1 are copied to LDS with direct buffer-to-LDS loads while tile k is in the
// MFMAs, so the tile loop waits on HBM only when a tile's compute is shorter than its loads.
// Vector memory operations complete in issue order, so each tile waits for its loads before
// issuing its stores, and the barriers order LDS only: no wait ever covers a tile's stores.
#include "rglru_launch.h"
#include "rglru_mfma.h"

namespace rglru {

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
constexpr int kWord3 = 0x00020000;  // buffer descriptor word 3: raw 32-bit data, no swizzle
constexpr uint32_t kLoPair = 0x05040100u, kHiPair = 0x07060302u;  // low / high halves
constexpr int kRows = 64;                                          // rows per tile

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

}  // namespace

template <int DH> struct PreTile {
  static constexpr int kGPW = 1;                         // 32-channel groups per wave
  static constexpr int kNW = DH / (32 * kGPW);           // waves (two per SIMD at Dh = 256)
  static constexpr int kThreads = 64 * kNW;
  static constexpr int kKS = DH / 16;        // MFMA k-steps
  static constexpr int kLda = DH + 8;        // bf16 A-tile row stride
  static constexpr int kRowsPerLoad = 1024 / (2 * DH);  // x rows per wave-wide 16 B/lane load
  static constexpr int kLoads = (kRows + 3 + kRowsPerLoad - 1) / kRowsPerLoad;
  static constexpr int kXRows = kLoads * kRowsPerLoad;  // staged rows: tile + 3-row halo
};

// pre[b][t][g*DH + o] = fp16 pair (pa, px) for the tiles j = blockIdx.x / H, + per, ... of head
// g = blockIdx.x % H (tile j: sequence j % B, rows (j / B) * 64 ...). SPLIT: the conv output
// enters as bf16 hi + lo (the backward's recompute); otherwise as one bf16 operand, the rounding
// of the forward plans.
template <int DH, bool SPLIT>
__global__ __launch_bounds__(PreTile<DH>::kThreads, 2) void tile_preacts(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ conv_w,
    const bf16_t *__restrict__ W_a, const float *__restrict__ b_a,
    const bf16_t *__restrict__ W_x, const float *__restrict__ b_x, uint32_t *__restrict__ pre,
    int B, int T, int D, int H, int per) {
  typedef PreTile<DH> F;
  constexpr int PP = DH / 2;
  constexpr int kParts = SPLIT ? 2 : 1;
  __shared__ __attribute__((aligned(16))) bf16_t xa[kParts * kRows * F::kLda];  // [hi, lo] conv out
  __shared__ __attribute__((aligned(16))) bf16_t xr[F::kXRows * DH];       // staged x rows
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lrow = lane & 31;
  const int half = lane >> 5;
  const int g = blockIdx.x % H;
  const int nTT = (T + kRows - 1) / kRows;
  const int ntiles = B * nTT;
  // this lane's output channels: cl0 + 32 gi, gi < kGPW
  const int cl0 = w * 32 * F::kGPW + lrow;
  float ba[F::kGPW], bx[F::kGPW];
  bf16x8_t wa[F::kGPW][F::kKS], wx[F::kGPW][F::kKS];
#pragma unroll
  for (int gi = 0; gi < F::kGPW; ++gi) {
    const int cl = cl0 + 32 * gi;
    ba[gi] = b_a[g * DH + cl];
    bx[gi] = b_x[g * DH + cl];
    const bf16_t *ra = W_a + (static_cast<size_t>(g) * DH + cl) * DH + half * 8;
    const bf16_t *rx = W_x + (static_cast<size_t>(g) * DH + cl) * DH + half * 8;
#pragma unroll
    for (int ks = 0; ks < F::kKS; ++ks) {
      wa[gi][ks] = load_bf16x8(ra + ks * 16);
      wx[gi][ks] = load_bf16x8(rx + ks * 16);
    }
  }
  // conv role: channel pair pc (taps as bf16 pairs (w0, w1), (w2, w3)), rows pr0 .. pr0+PRPG-1
  constexpr int PRPG = kRows * PP / F::kThreads;
  const int pc = tid % PP;
  const int pr0 = (tid / PP) * PRPG;
  bf16x2_t w01l, w23l, w01h, w23h;
  {
    uint32_t cw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      cw[k] = *reinterpret_cast<const uint32_t *>(conv_w + static_cast<size_t>(k) * D + g * DH +
                                                 2 * pc);
    w01l = as_bf16x2(__builtin_amdgcn_perm(cw[1], cw[0], kLoPair));
    w23l = as_bf16x2(__builtin_amdgcn_perm(cw[3], cw[2], kLoPair));
    w01h = as_bf16x2(__builtin_amdgcn_perm(cw[1], cw[0], kHiPair));
    w23h = as_bf16x2(__builtin_amdgcn_perm(cw[3], cw[2], kHiPair));
  }
  // Staging of tile j's rows t0-3 .. t0+63 (+ a few unused) by all waves: the buffer covers
  // exactly sequence b, so its range check returns zeros before t = 0 and past T - 1.
  constexpr int kLanesPerRow = DH / 8;
  const unsigned lane_off =
      static_cast<unsigned>((lane / kLanesPerRow) * 2 * D + g * DH * 2 + (lane % kLanesPerRow) * 16);
  auto stage = [&](int j) {
    const int b = j % B, t0 = (j / B) * kRows;
    const __amdgpu_buffer_rsrc_t seq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(x + static_cast<size_t>(b) * T * D), static_cast<short>(0),
        rec_bytes(T, D, 2u), kWord3);
    for (int i = w; i < F::kLoads; i += F::kNW) {
      const unsigned row_off = row_bytes(t0 - 3 + i * F::kRowsPerLoad, D, 2u);
      dma_16b(seq, row_off + lane_off, lds_addr(xr + i * F::kRowsPerLoad * DH));
    }
  };
  int j = blockIdx.x / H;
  if (j < ntiles) stage(j);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): own staging loads landed
  // The barriers order LDS only: the staging loads are waited for explicitly (before the
  // stores), so no barrier waits for the previous tile's stores.
  for (; j < ntiles; j += per) {
    lds_barrier();  // staged rows visible; xa free
    // ---- conv (fp32 dot products of bf16 pairs) -> hi / lo bf16
#pragma unroll 4
    for (int r = 0; r < PRPG; ++r) {
      const int row = pr0 + r;  // tile row; staged row row + k holds time t0 - 3 + row + k
      uint32_t xv[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) xv[k] = *reinterpret_cast<const uint32_t *>(xr + (row + k) * DH + 2 * pc);
      const float o0 = __builtin_amdgcn_fdot2_f32_bf16(
          as_bf16x2(__builtin_amdgcn_perm(xv[3], xv[2], kLoPair)), w23l,
          __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(__builtin_amdgcn_perm(xv[1], xv[0], kLoPair)),
                                          w01l, 0.0f, false),
          false);
      const float o1 = __builtin_amdgcn_fdot2_f32_bf16(
          as_bf16x2(__builtin_amdgcn_perm(xv[3], xv[2], kHiPair)), w23h,
          __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(__builtin_amdgcn_perm(xv[1], xv[0], kHiPair)),
                                          w01h, 0.0f, false),
          false);
      const uint32_t hv = pack_bf16x2(o0, o1);
      *reinterpret_cast<uint32_t *>(xa + row * F::kLda + 2 * pc) = hv;
      if constexpr (SPLIT)
        *reinterpret_cast<uint32_t *>(xa + (kRows + row) * F::kLda + 2 * pc) =
            pack_bf16x2(o0 - bf16lo(hv), o1 - bf16hi(hv));
    }
    lds_barrier();  // xa ready; xr free
    const int jn = j + per;
    if (jn < ntiles) stage(jn);
    // ---- [64 x DH] x [DH x 2 DH]: A = hi (+ lo)
    f32x16_t acc[F::kGPW][2][2];  // [group][row tile][gate]
#pragma unroll
    for (int gi = 0; gi < F::kGPW; ++gi)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) acc[gi][rt][0] = acc[gi][rt][1] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < F::kKS; ++ks)
#pragma unroll
      for (int part = 0; part < kParts; ++part)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const bf16x8_t af =
              load_bf16x8(xa + (part * kRows + rt * 32 + lrow) * F::kLda + ks * 16 + half * 8);
#pragma unroll
          for (int gi = 0; gi < F::kGPW; ++gi) {
            acc[gi][rt][0] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, wa[gi][ks], acc[gi][rt][0], 0, 0, 0);
            acc[gi][rt][1] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, wx[gi][ks], acc[gi][rt][1], 0, 0, 0);
          }
        }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // next tile's staging landed
    // ---- bias, fp16 pairs, store, through a buffer descriptor over sequence b's pre-activations:
    // a wave-uniform row offset plus this lane's byte offset (its channel and its half's 4-row
    // shift), one 32-bit add per store; the range check drops rows past T (no per-row branch).
    // Dv is re-read through an empty asm each tile so that the 32 row offsets are not hoisted
    // out of the loop into registers.
    const int b = j % B, t0 = (j / B) * kRows;
    unsigned Dv = static_cast<unsigned>(D);
    asm volatile("" : "+s"(Dv));
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        pre + static_cast<size_t>(b) * T * D, static_cast<short>(0), rec_bytes(T, D, 4u), kWord3);
#pragma unroll
    for (int gi = 0; gi < F::kGPW; ++gi) {
      const unsigned lane_off =
          (static_cast<unsigned>(g * DH + cl0 + 32 * gi) + 4u * half * Dv) * 4u;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int r = rt * 32 + 8 * (jj >> 2) + (jj & 3);  // half 0's row; half 1: 4 further
          __builtin_amdgcn_raw_buffer_store_b32(
              pack_f16x2(acc[gi][rt][0][jj] + ba[gi], acc[gi][rt][1][jj] + bx[gi]), rp,
              static_cast<int>(static_cast<unsigned>(t0 + r) * Dv * 4u + lane_off), 0, 0);
        }
    }
  }
}

// The rest of the backward for the tiles of head g, one 64-step tile at a time and nothing per
// element written but dx: dxc = (its direct part, fp16 from the per-element pass) + sum_k dp[k]
// wti[g][i][k] (fp16 MFMA, Wt resident), then the conv's transpose dx[t] = sum_j w_j dxc[t+3-j]
// and the tile's partial sums dconv_w[j] += dxc[t] x[t-3+j]. dx of the tile's rows needs dxc of
// the next three rows, so each tile computes dxc for 67 rows -- its own and three of the next
// tile -- with one more pass of MFMAs over a 32-row tile of which three rows are kept (half as
// many again MFMAs, no dependence between tiles and no dxc in HBM).
// dp rows (fp16 pairs, dpa low) are staged one row per load instruction into rows padded by 16
// bytes, so the A-operand reads of 32 rows fall on distinct banks; two tile buffers, tile k+1
// loading while tile k is in the MFMAs. Per tile: [barrier] stage tile k+1, load the direct
// part (16 bytes per lane, row-major), MFMAs, [barrier] the products (fp32) over the tile's own
// dp buffer, [barrier] + direct part, [barrier] dx and the dconv_w sums (thread = channel pair x
// 16 rows, x read 4 bytes per lane), [barrier] the sums over the four row blocks. The LDS detour
// turns the accumulator layout (one channel per lane, rows 4 apart) into rows. Vector memory
// completes in issue order and the barriers order LDS only.
template <int DH> struct DxcTile {
  static_assert(DH == 128 || DH == 256, "resident dxc tile needs Dh in {128, 256}");
  static constexpr int kGPW = 1;          // 32-channel groups per wave
  static constexpr int kNW = DH / (32 * kGPW);
  static constexpr int kThreads = 64 * kNW;
  static constexpr int K = 2 * DH;
  static constexpr int kKS = K / 16;
  static constexpr int kLd = K + 8;            // fp16 row stride (row bytes + 16)
  static constexpr int kLanesPerRow = K / 8;   // 16-byte pieces per row (<= 64)
  static constexpr int kRowsX = kRows + 3;     // the tile and the next tile's first three rows
  static constexpr int kLdo = DH + 4;          // fp32 row stride of the dxc rows
  static constexpr int kPieces = kRowsX * DH / 8;                           // 16-byte pieces
  static constexpr int kPer = (kPieces + kThreads - 1) / kThreads;          // per thread
  static constexpr int kRB = kThreads / (DH / 2);  // row blocks of the conv's transpose (4)
  static constexpr int kRBRows = kRows / kRB;      // 16
  static_assert(kRowsX * kLdo * 4 == kRowsX * kLd * 2, "dxc rows fill one dp buffer");
  static_assert(kRB == 4, "four row blocks");
};

template <int DH>
__global__ __launch_bounds__(DxcTile<DH>::kThreads, 2) void tile_dxc(
    const uint32_t *__restrict__ dp, const uint16_t *__restrict__ wti,
    const uint16_t *__restrict__ dxd, const bf16_t *__restrict__ x,
    const bf16_t *__restrict__ conv_w, bf16_t *__restrict__ dx, float *__restrict__ pcw, int B,
    int T, int D, int H, int per) {
  typedef DxcTile<DH> F;
  __shared__ __attribute__((aligned(16))) uint16_t la[2 * F::kRowsX * F::kLd];
  __shared__ float red[F::kRB * 4 * DH];  // [row block][tap][channel] partial sums
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lrow = lane & 31;
  const int half = lane >> 5;
  const int g = blockIdx.x % H;
  const int nTT = (T + kRows - 1) / kRows;
  const int ntiles = B * nTT;
  const int ci0 = w * 32 * F::kGPW + lrow;  // output channels ci0 + 32 gi within the head
  f16x8_t wr[F::kGPW][F::kKS];
#pragma unroll
  for (int gi = 0; gi < F::kGPW; ++gi) {
    const uint16_t *row = wti + (static_cast<size_t>(g) * DH + ci0 + 32 * gi) * F::K + half * 8;
#pragma unroll
    for (int ks = 0; ks < F::kKS; ++ks) wr[gi][ks] = load_f16x8(row + ks * 16);
  }
  // the conv's transpose: thread = channel pair pc (channels 2 pc, 2 pc + 1), rows rb * 16 ..
  const int pc = tid % (DH / 2), rb = tid / (DH / 2);
  float cw[4][2];  // taps of the two channels
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t v = *reinterpret_cast<const uint32_t *>(conv_w + static_cast<size_t>(j) * D +
                                                           g * DH + 2 * pc);
    cw[j][0] = bf16lo(v);
    cw[j][1] = bf16hi(v);
  }
  // staging: tile row r (0 .. kRowsX - 1) by wave r % kNW, lanes 0 .. kLanesPerRow-1; rows past
  // T read zeros
  const bool slane = lane < F::kLanesPerRow;
  auto stage = [&](int j, int buf) {
    const int b = j % B, t0 = (j / B) * kRows;
    const __amdgpu_buffer_rsrc_t seq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t *>(dp + static_cast<size_t>(b) * T * D), static_cast<short>(0),
        rec_bytes(T, D, 4u), kWord3);
    if (slane) {
      for (int r = w; r < F::kRowsX; r += F::kNW) {
        const unsigned off = row_bytes(t0 + r, D, 4u) + static_cast<unsigned>(g * DH * 4 + lane * 16);
        dma_16b(seq, off, lds_addr(la + (buf * F::kRowsX + r) * F::kLd));
      }
    }
  };
  int j = blockIdx.x / H;
  if (j < ntiles) stage(j, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  for (int it = 0; j < ntiles; j += per, ++it) {
    // this tile's rows are in buffer it & 1; the other buffer's readers (the previous tile's
    // MFMAs and dxc reads) are past this barrier
    lds_barrier();
    const int jn = j + per;
    if (jn < ntiles) stage(jn, (it + 1) & 1);
    const int b = j % B, t0 = (j / B) * kRows;
    // Sequence b of dxd, x and dx through buffer descriptors: a row's byte offset is
    // wave-uniform, a lane's a fixed 32-bit add, and the range check returns zeros for rows
    // before t = 0 (negative offsets wrap past the end) or past T - 1 and drops stores there.
    const __amdgpu_buffer_rsrc_t sd = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(dxd + static_cast<size_t>(b) * T * D), static_cast<short>(0),
        rec_bytes(T, D, 2u), kWord3);
    const __amdgpu_buffer_rsrc_t sx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(x + static_cast<size_t>(b) * T * D), static_cast<short>(0),
        rec_bytes(T, D, 2u), kWord3);
    const __amdgpu_buffer_rsrc_t so = __builtin_amdgcn_make_buffer_rsrc(
        dx + static_cast<size_t>(b) * T * D, static_cast<short>(0), rec_bytes(T, D, 2u), kWord3);
    // the direct part of dxc of rows t0 .. t0 + 66, 16 bytes (8 channels) per lane and piece
    // (pieces past the 67 rows read nothing: their offset is out of range)
    u32x4_t dv[F::kPer];
#pragma unroll
    for (int q = 0; q < F::kPer; ++q) {
      const int idx = tid + q * F::kThreads, r = idx / (DH / 8), c8 = idx % (DH / 8);
      const unsigned off = idx < F::kPieces
                               ? row_bytes(t0 + r, D, 2u) + static_cast<unsigned>(g * DH + 8 * c8) * 2u
                               : 0x80000000u;
      dv[q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                              sd, static_cast<int>(off), 0, 0));
    }
    const uint16_t *lt = la + (it & 1) * F::kRowsX * F::kLd;
    f32x16_t acc[F::kGPW][3];  // row tiles: rows 0-31, 32-63, 64-95 (of which 64-66 are kept)
#pragma unroll
    for (int gi = 0; gi < F::kGPW; ++gi) acc[gi][0] = acc[gi][1] = acc[gi][2] = f32x16_t{};
    const int rx = min(64 + lrow, F::kRowsX - 1);  // the third tile's row (clamped: not kept)
#pragma unroll
    for (int ks = 0; ks < F::kKS; ++ks)
#pragma unroll
      for (int rt = 0; rt < 3; ++rt) {
        const int row = rt < 2 ? rt * 32 + lrow : rx;
        const f16x8_t af = load_f16x8(lt + row * F::kLd + ks * 16 + half * 8);
#pragma unroll
        for (int gi = 0; gi < F::kGPW; ++gi)
          acc[gi][rt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, wr[gi][ks], acc[gi][rt], 0, 0, 0);
      }
    // the products, row-major in fp32, over this tile's dp rows
    float *po = reinterpret_cast<float *>(la + (it & 1) * F::kRowsX * F::kLd);
    lds_barrier();  // every wave is done with this tile's dp rows
#pragma unroll
    for (int gi = 0; gi < F::kGPW; ++gi)
#pragma unroll
      for (int rt = 0; rt < 3; ++rt)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int r = rt * 32 + 8 * (jj >> 2) + 4 * half + (jj & 3);
          if (rt < 2 || r < F::kRowsX) po[r * F::kLdo + ci0 + 32 * gi] = acc[gi][rt][jj];
        }
    // x rows t0 + 16 rb - 3 .. t0 + 16 rb + 15 of this thread's channel pair (the dconv_w sums),
    // in flight while the products and the direct part are added
    uint32_t xw[F::kRBRows + 3];
    const unsigned pair_off = static_cast<unsigned>(g * DH + 2 * pc) * 2u;
#pragma unroll
    for (int k = 0; k < F::kRBRows + 3; ++k)
      xw[k] = __builtin_amdgcn_raw_buffer_load_b32(
          sx, static_cast<int>(row_bytes(t0 + rb * F::kRBRows - 3 + k, D, 2u) + pair_off), 0, 0);
    lds_barrier();  // products complete
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): next tile's staging, direct part, x rows
#pragma unroll
    for (int q = 0; q < F::kPer; ++q) {
      const int idx = tid + q * F::kThreads, r = idx / (DH / 8), c8 = idx % (DH / 8);
      if (idx < F::kPieces) {
        float4 *pp = reinterpret_cast<float4 *>(po + r * F::kLdo + 8 * c8);
        float4 p0 = pp[0], p1 = pp[1];
        p0.x += f16lo(dv[q][0]);
        p0.y += f16hi(dv[q][0]);
        p0.z += f16lo(dv[q][1]);
        p0.w += f16hi(dv[q][1]);
        p1.x += f16lo(dv[q][2]);
        p1.y += f16hi(dv[q][2]);
        p1.z += f16lo(dv[q][3]);
        p1.w += f16hi(dv[q][3]);
        pp[0] = p0;
        pp[1] = p1;
      }
    }
    lds_barrier();  // dxc of the 67 rows complete
    // dx[t] = sum_j w_j dxc[t + 3 - j] over this thread's 16 rows; dconv_w[j] += dxc[t] x[t-3+j]
    {
      float s[4][2] = {};
      const float *pr = po + 2 * pc;
      float2 gw[4];  // dxc rows r .. r + 3
#pragma unroll
      for (int k = 0; k < 3; ++k)
        gw[k + 1] = *reinterpret_cast<const float2 *>(pr + (rb * F::kRBRows + k) * F::kLdo);
#pragma unroll
      for (int u = 0; u < F::kRBRows; ++u) {
        const int r = rb * F::kRBRows + u;
        gw[0] = gw[1];
        gw[1] = gw[2];
        gw[2] = gw[3];
        gw[3] = *reinterpret_cast<const float2 *>(pr + (r + 3) * F::kLdo);
        const float v0 = fmaf(cw[0][0], gw[3].x, fmaf(cw[1][0], gw[2].x,
                                                      fmaf(cw[2][0], gw[1].x, cw[3][0] * gw[0].x)));
        const float v1 = fmaf(cw[0][1], gw[3].y, fmaf(cw[1][1], gw[2].y,
                                                      fmaf(cw[2][1], gw[1].y, cw[3][1] * gw[0].y)));
        __builtin_amdgcn_raw_buffer_store_b32(
            pack_bf16x2(v0, v1), so, static_cast<int>(row_bytes(t0 + r, D, 2u) + pair_off), 0, 0);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {  // x[t - 3 + jt] is xw[u + jt]
          s[jt][0] = fmaf(gw[0].x, bf16lo(xw[u + jt]), s[jt][0]);
          s[jt][1] = fmaf(gw[0].y, bf16hi(xw[u + jt]), s[jt][1]);
        }
      }
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
        *reinterpret_cast<float2 *>(red + (rb * 4 + jt) * DH + 2 * pc) = make_float2(s[jt][0], s[jt][1]);
    }
    lds_barrier();  // row-block sums ready
    // the tile's dconv_w partial sums, in a fixed order: pcw[b][tile][j][d]
    for (int i = tid; i < 4 * DH; i += F::kThreads) {
      const int jt = i / DH, c = i % DH;
      float v = 0.0f;
#pragma unroll
      for (int q = 0; q < F::kRB; ++q) v += red[(q * 4 + jt) * DH + c];
      pcw[((static_cast<size_t>(b) * nTT + t0 / kRows) * 4 + jt) * D + g * DH + c] = v;
    }
  }
}

// ---- launchers ---------------------------------------------------------------------------------
namespace {
int cu_count() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return cus;
}
}  // namespace

bool resident_preacts_supported(int Dh) { return Dh == 32 || Dh == 64 || Dh == 128 || Dh == 256; }
bool resident_dxc_supported(int Dh) { return Dh == 128 || Dh == 256; }

hipError_t launch_resident_preacts(const void *x, const void *conv_w, const void *W_a,
                                   const float *b_a, const void *W_x, const float *b_x,
                                   void *pre, int B, int T, int D, int H, hipStream_t s,
                                   bool split) {
  // one workgroup per CU (the LDS of a tile), the same number for every head
  const int per = std::max(1, cu_count() / H);
  const bf16_t *xx = static_cast<const bf16_t *>(x);
  const bf16_t *cw = static_cast<const bf16_t *>(conv_w);
  const bf16_t *wa = static_cast<const bf16_t *>(W_a);
  const bf16_t *wx = static_cast<const bf16_t *>(W_x);
  uint32_t *pp = static_cast<uint32_t *>(pre);
  switch (D / H) {
#define RGLRU_PRE_CASE(DHV)                                                                       \
  case DHV:                                                                                       \
    if (split)                                                                                    \
      tile_preacts<DHV, true><<<H * per, PreTile<DHV>::kThreads, 0, s>>>(xx, cw, wa, b_a, wx, b_x, \
                                                                         pp, B, T, D, H, per);    \
    else                                                                                          \
      tile_preacts<DHV, false><<<H * per, PreTile<DHV>::kThreads, 0, s>>>(                        \
          xx, cw, wa, b_a, wx, b_x, pp, B, T, D, H, per);                                         \
    break;
    RGLRU_PRE_CASE(32)
    RGLRU_PRE_CASE(64)
    RGLRU_PRE_CASE(128)
    RGLRU_PRE_CASE(256)
#undef RGLRU_PRE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_resident_dxc(const void *dp, const void *wti, const uint16_t *dxd,
                               const void *x, const void *conv_w, void *dx, float *pcw, int B,
                               int T, int D, int H, hipStream_t s) {
  const int per = std::max(1, cu_count() / H);
  const uint32_t *p = static_cast<const uint32_t *>(dp);
  const uint16_t *wt = static_cast<const uint16_t *>(wti);
  const bf16_t *xx = static_cast<const bf16_t *>(x);
  const bf16_t *cw = static_cast<const bf16_t *>(conv_w);
  bf16_t *dd = static_cast<bf16_t *>(dx);
  switch (D / H) {
    case 128:
      tile_dxc<128><<<H * per, DxcTile<128>::kThreads, 0, s>>>(p, wt, dxd, xx, cw, dd, pcw, B, T,
                                                                D, H, per);
      break;
    case 256:
      tile_dxc<256><<<H * per, DxcTile<256>::kThreads, 0, s>>>(p, wt, dxd, xx, cw, dd, pcw, B, T,
                                                                D, H, per);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rglru
