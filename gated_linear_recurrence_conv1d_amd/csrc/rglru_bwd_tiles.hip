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
        const_cast<bf16_t *>(x + static_cast<size_t>(b) * T * D), static_cast<short>(0), T * D * 2,
        kWord3);
    for (int i = w; i < F::kLoads; i += F::kNW) {
      const unsigned row_off = static_cast<unsigned>((t0 - 3 + i * F::kRowsPerLoad) * 2 * D);
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
    // ---- bias, fp16 pairs, store. Row addresses: a wave-uniform row pointer plus this lane's
    // byte offset (its channel and its half's 4-row shift); Dv is re-read through an empty asm
    // each tile so that the 32 row offsets are not hoisted out of the loop into registers.
    const int b = j % B, t0 = (j / B) * kRows;
    unsigned Dv = static_cast<unsigned>(D);
    asm volatile("" : "+s"(Dv));
    const char *tile = reinterpret_cast<const char *>(pre + (static_cast<size_t>(b) * T + t0) * D +
                                                      g * DH);
    const bool full = t0 + kRows <= T;
#pragma unroll
    for (int gi = 0; gi < F::kGPW; ++gi) {
      const unsigned lane_off = (static_cast<unsigned>(cl0 + 32 * gi) + 4u * half * Dv) * 4u;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int r = rt * 32 + 8 * (jj >> 2) + (jj & 3);  // half 0's row; half 1: 4 further
          if (full || t0 + r + 4 * half < T)
            *reinterpret_cast<uint32_t *>(const_cast<char *>(tile) + static_cast<size_t>(r) * Dv * 4u +
                                          lane_off) =
                pack_f16x2(acc[gi][rt][0][jj] + ba[gi], acc[gi][rt][1][jj] + bx[gi]);
        }
    }
  }
}

// dxc[b][t][g*DH + i] += sum_k dp[b][t][g*DH .. as 2 DH fp16][k] wti[g][i][k] for the tiles of
// head g, as above (fp16 operands, dxc in fp16). dp rows (fp16 pairs, dpa low) are staged one row
// per load instruction into rows padded by 16 bytes, so the A-operand reads of 32 rows fall on
// distinct banks; two tile buffers, tile k+1 loading while tile k is in the MFMAs. Per tile:
// [barrier] stage tile k+1, load this tile's dxc (16 bytes per lane, row-major), MFMAs,
// [barrier] the products into the tile's own dp buffer (fp32, now free), [barrier] one wait
// (vmcnt(0): staging and dxc loads), then dxc + product stored 16 bytes per lane. The detour
// through the LDS turns the accumulator layout (one channel per lane, rows 4 apart) into
// row-major pieces: stored straight from the accumulators, fp16 dxc went out as 2-byte stores
// (half of a 128-byte line per wave) and took twice as long. Vector memory completes in issue
// order, so the wait sits before this tile's stores and the barriers order LDS only.
template <int DH> struct DxcTile {
  static_assert(DH == 128 || DH == 256, "resident dxc tile needs Dh in {128, 256}");
  static constexpr int kGPW = 1;          // 32-channel groups per wave
  static constexpr int kNW = DH / (32 * kGPW);
  static constexpr int kThreads = 64 * kNW;
  static constexpr int K = 2 * DH;
  static constexpr int kKS = K / 16;
  static constexpr int kLd = K + 8;            // fp16 row stride (row bytes + 16)
  static constexpr int kLanesPerRow = K / 8;   // 16-byte pieces per row (<= 64)
};

template <int DH>
__global__ __launch_bounds__(DxcTile<DH>::kThreads, 2) void tile_dxc(
    const uint32_t *__restrict__ dp, const uint16_t *__restrict__ wti, uint16_t *__restrict__ dxc,
    int B, int T, int D, int H, int per) {
  typedef DxcTile<DH> F;
  __shared__ __attribute__((aligned(16))) uint16_t la[2 * kRows * F::kLd];
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
  // staging: tile row r by wave r % kNW, lanes 0 .. kLanesPerRow-1; rows past T read zeros
  const bool slane = lane < F::kLanesPerRow;
  auto stage = [&](int j, int buf) {
    const int b = j % B, t0 = (j / B) * kRows;
    const __amdgpu_buffer_rsrc_t seq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t *>(dp + static_cast<size_t>(b) * T * D), static_cast<short>(0),
        T * D * 4, kWord3);
    if (slane) {
      for (int r = w; r < kRows; r += F::kNW) {
        const unsigned off = static_cast<unsigned>(((t0 + r) * D + g * DH) * 4 + lane * 16);
        dma_16b(seq, off, lds_addr(la + (buf * kRows + r) * F::kLd));
      }
    }
  };
  int j = blockIdx.x / H;
  if (j < ntiles) stage(j, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  for (int it = 0; j < ntiles; j += per, ++it) {
    // this tile's rows are in buffer it & 1; the other buffer's readers (the previous tile's
    // MFMAs and product reads) are past this barrier
    lds_barrier();
    // the next tile's rows, then the dxc values this lane updates (neither depends on the MFMAs;
    // both land while they run)
    const int jn = j + per;
    if (jn < ntiles) stage(jn, (it + 1) & 1);
    const int b = j % B, t0 = (j / B) * kRows;
    // this tile's dxc values, 16 bytes (8 channels) per lane and piece, rows past T as zeros
    constexpr int kPieces = kRows * DH / 8;
    constexpr int kPer = kPieces / F::kThreads;
    static_assert(kPieces % F::kThreads == 0, "pieces per thread");
    uint16_t *tile = dxc + (static_cast<size_t>(b) * T + t0) * D + g * DH;
    u32x4_t dv[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int idx = tid + q * F::kThreads, r = idx / (DH / 8), c8 = idx % (DH / 8);
      dv[q] = t0 + r < T ? *reinterpret_cast<const u32x4_t *>(tile + static_cast<size_t>(r) * D + 8 * c8)
                         : u32x4_t{0u, 0u, 0u, 0u};
    }
    const uint16_t *lt = la + (it & 1) * kRows * F::kLd;
    f32x16_t acc[F::kGPW][2];
#pragma unroll
    for (int gi = 0; gi < F::kGPW; ++gi) acc[gi][0] = acc[gi][1] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < F::kKS; ++ks)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const f16x8_t af = load_f16x8(lt + (rt * 32 + lrow) * F::kLd + ks * 16 + half * 8);
#pragma unroll
        for (int gi = 0; gi < F::kGPW; ++gi)
          acc[gi][rt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, wr[gi][ks], acc[gi][rt], 0, 0, 0);
      }
    // the products, row-major in fp32, over this tile's dp rows (kRows x (DH + 4) floats: the
    // same bytes as kRows x kLd fp16)
    constexpr int kLdo = DH + 4;
    static_assert(kRows * kLdo * 4 == kRows * F::K * 2 + kRows * 16, "product tile fits");
    float *po = reinterpret_cast<float *>(la + (it & 1) * kRows * F::kLd);
    lds_barrier();  // every wave is done with this tile's dp rows
#pragma unroll
    for (int gi = 0; gi < F::kGPW; ++gi)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
          po[(rt * 32 + 8 * (jj >> 2) + 4 * half + (jj & 3)) * kLdo + ci0 + 32 * gi] = acc[gi][rt][jj];
    lds_barrier();  // products complete
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): next tile's staging and the dxc values
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int idx = tid + q * F::kThreads, r = idx / (DH / 8), c8 = idx % (DH / 8);
      if (t0 + r < T) {
        const float4 p0 = *reinterpret_cast<const float4 *>(po + r * kLdo + 8 * c8);
        const float4 p1 = *reinterpret_cast<const float4 *>(po + r * kLdo + 8 * c8 + 4);
        u32x4_t o;
        o[0] = pack_f16x2(f16lo(dv[q][0]) + p0.x, f16hi(dv[q][0]) + p0.y);
        o[1] = pack_f16x2(f16lo(dv[q][1]) + p0.z, f16hi(dv[q][1]) + p0.w);
        o[2] = pack_f16x2(f16lo(dv[q][2]) + p1.x, f16hi(dv[q][2]) + p1.y);
        o[3] = pack_f16x2(f16lo(dv[q][3]) + p1.z, f16hi(dv[q][3]) + p1.w);
        *reinterpret_cast<u32x4_t *>(tile + static_cast<size_t>(r) * D + 8 * c8) = o;
      }
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

hipError_t launch_resident_dxc(const void *dp, const void *wti, uint16_t *dxc, int B, int T, int D,
                               int H, hipStream_t s) {
  const int per = std::max(1, cu_count() / H);
  const uint32_t *p = static_cast<const uint32_t *>(dp);
  const uint16_t *wt = static_cast<const uint16_t *>(wti);
  switch (D / H) {
    case 128: tile_dxc<128><<<H * per, DxcTile<128>::kThreads, 0, s>>>(p, wt, dxc, B, T, D, H, per); break;
    case 256: tile_dxc<256><<<H * per, DxcTile<256>::kThreads, 0, s>>>(p, wt, dxc, B, T, D, H, per); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rglru
