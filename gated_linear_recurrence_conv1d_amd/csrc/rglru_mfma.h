// rglru_mfma.h -- the block-diagonal gate projection as a bf16 MFMA tile on gfx950.
//
// The gates do not read the recurrent state (alby13 blog, "Core Components of Griffin -- 1.
// RG-LRU"), so for every head g they form one dense contraction over all (b, t) rows:
//   [pa | px][rows x 2Dh] = xc[rows x Dh] * [W_a[g] ; W_x[g]]^T,
// the only dense contraction on the path. One workgroup owns a 64-row tile of one head and all
// 2*Dh output columns, so the conv that produces xc is computed once per tile.
//
// Tile mapping: 4 waves; the 64 rows are two 32-row MFMA tiles, the Dh channels are Dh/32
// groups of 32. Each wave owns (groups x row tiles) and, for every group, BOTH gates -- so the
// pa and px of one (row, channel) land in the same lane and the same accumulator slot.
// v_mfma_f32_32x32x16_bf16: lane l feeds row/column l % 32 with 8 consecutive k values from
// k-half l / 32; A and B use the same k order, so the contraction is exact in any k order.
// Accumulator j of lane l is C[8 (j/4) + 4 (l/32) + (j%4)][l % 32].
#pragma once

#include "rglru_device.h"

namespace rglru {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTileRows = 64;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int DH> struct GateTile {
  static_assert(DH == 32 || DH == 64 || DH == 128 || DH == 256,
                "MFMA gate tile needs Dh in {32, 64, 128, 256}");
  static constexpr int kGroups = DH / 32;
  static constexpr int kRPW = DH >= 128 ? 2 : 1;                 // row tiles per wave
  static constexpr int kGPW = DH >= 128 ? kGroups / kWaves : 1;  // channel groups per wave
  static constexpr int kLda = DH + 8;  // LDS row stride in bf16 (16 B pad against conflicts)
  // First group and first row tile of wave w; `active` is false for waves with no work.
  __device__ static void assign(int w, int &g0, int &r0, bool &active) {
    if (kRPW == 2) {
      g0 = w * kGPW;
      r0 = 0;
    } else {
      g0 = w >> 1;
      r0 = w & 1;
    }
    active = g0 < kGroups;
  }
  // Row (within the 64-row tile) of accumulator j in lane l for row tile rt.
  __device__ static int acc_row(int rt, int j, int lane) {
    return rt * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
  }
};

__device__ __forceinline__ bf16x8_t load_bf16x8(const bf16_t *p) {
  u32x4_t v = *reinterpret_cast<const u32x4_t *>(p);
  return __builtin_bit_cast(bf16x8_t, v);
}

// fp16 operands (v_mfma_f32_32x32x16_f16: the same lane layout as the bf16 instruction), held as
// raw 16-bit words in memory.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f16x8_t load_f16x8(const uint16_t *p) {
  u32x4_t v = *reinterpret_cast<const u32x4_t *>(p);
  return __builtin_bit_cast(f16x8_t, v);
}

// acc[gi][ri][gate] = A(rows of row tile r0+ri) * W_gate(rows of group g0+gi)^T over k = 0..DH.
// lds_a: [64][kLda] bf16 conv output of the tile. Wa_g / Wx_g: this head's [DH][DH] weights.
// SPLIT: lds_lo holds the bf16 residual of the conv output (xc - hi) and A = hi + lo, which makes
// the contraction accurate to about 2^-16 of its terms instead of 2^-9 (the weights are exact).
template <int DH, bool SPLIT = false>
__device__ __forceinline__ void gate_tile_mfma(const bf16_t *lds_a, const bf16_t *Wa_g,
                                               const bf16_t *Wx_g, int g0, int r0, int lane,
                                               f32x16_t (&acc)[GateTile<DH>::kGPW]
                                                              [GateTile<DH>::kRPW][2],
                                               const bf16_t *lds_lo = nullptr) {
  typedef GateTile<DH> C;
  constexpr int kParts = SPLIT ? 2 : 1;
  const int lrow = lane & 31;
  const int khalf = (lane >> 5) * 8;
#pragma unroll
  for (int gi = 0; gi < C::kGPW; ++gi)
#pragma unroll
    for (int ri = 0; ri < C::kRPW; ++ri) {
      acc[gi][ri][0] = f32x16_t{};
      acc[gi][ri][1] = f32x16_t{};
    }
#pragma unroll 2
  for (int k0 = 0; k0 < DH; k0 += 16) {
    bf16x8_t af[kParts][C::kRPW];
#pragma unroll
    for (int ri = 0; ri < C::kRPW; ++ri) {
      const int off = ((r0 + ri) * 32 + lrow) * C::kLda + k0 + khalf;
      af[0][ri] = load_bf16x8(lds_a + off);
      if constexpr (SPLIT) af[kParts - 1][ri] = load_bf16x8(lds_lo + off);
    }
    bf16x8_t bf[C::kGPW][2];
#pragma unroll
    for (int gi = 0; gi < C::kGPW; ++gi) {
      const size_t wrow = static_cast<size_t>((g0 + gi) * 32 + lrow) * DH + k0 + khalf;
      bf[gi][0] = load_bf16x8(Wa_g + wrow);
      bf[gi][1] = load_bf16x8(Wx_g + wrow);
    }
#pragma unroll
    for (int p = 0; p < kParts; ++p)
#pragma unroll
      for (int gi = 0; gi < C::kGPW; ++gi)
#pragma unroll
        for (int ri = 0; ri < C::kRPW; ++ri) {
          acc[gi][ri][0] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[p][ri], bf[gi][0], acc[gi][ri][0], 0, 0, 0);
          acc[gi][ri][1] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[p][ri], bf[gi][1], acc[gi][ri][1], 0, 0, 0);
        }
  }
}

}  // namespace rglru
