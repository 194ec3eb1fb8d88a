// rglru_fused.hip -- the whole forward in one pass over HBM: temporal Conv1D, block-diagonal gate
// projections on MFMA, log-space gate nonlinearity and the RG-LRU scan, reading x once and
// writing y once (4 bytes per element for bf16 I/O instead of 14 for the split design).
//
// Why: the scan is memory-bound and its HBM traffic is what matters (Soham De's Griffin thread,
// tweet on the Pallas kernel that optimises HBM accesses); the gates do not read the state
// (alby13 blog, "Core Components of Griffin -- 1. RG-LRU"), so they can be computed for a whole
// time tile at once; the recurrence is diagonal (Soham De's thread, tweet on S4D/LRU), so each
// channel is an independent first-order affine recurrence h -> a h + u, and affine maps compose
// associatively: (A2, U2) o (A1, U1) = (A2 A1, A2 U1 + U2).
//
// Work unit: one tile = 64 time steps x all Dh channels of one head of one sequence. Each head
// has its own ticket counter; its tiles are handed out in time-major order (tt, then b), so a
// tile only ever waits for tiles with smaller tickets of the same head, all of which have been
// claimed by running workgroups: forward progress does not depend on how the hardware schedules
// workgroups. Per tile:
//   1. conv in fp32 from the tile's x rows (3-row halo), staged in LDS during the previous tile,
//      into LDS (a bf16 copy as the MFMA A operand, an fp32 copy for the input term);
//   2. [64 x Dh] x [Dh x 2Dh] on v_mfma_f32_32x32x16_bf16, fp32 accumulators; the B operand is
//      this head's W_a / W_x rows, resident in registers for the kernel's life;
//   3. gates elementwise in the accumulator layout -> (a, u) per element;
//   4. scan inside the tile: the MFMA A operand's rows are permuted so that each lane holds two
//      runs of 16 consecutive steps of its channel, the lanes of the other half the two runs in
//      between; runs are scanned in-lane, their affine maps exchanged between the halves with
//      v_permlane32_swap and chained in every lane. Row tile 1's MFMAs are interleaved with
//      row tile 0's gate math;
//   5. decoupled look-back: publish the tile's aggregate (A, U) per channel, walk back over the
//      predecessor tiles of the same (sequence, head), combining aggregates until an inclusive
//      state (or the sequence start) is found, publish this tile's inclusive state;
//   6. fix-up h_t = P_t * carry + S_t and store y (and h_T for the last tile).
// Each (tile, channel) has one 64-bit word, written and read with relaxed agent-scope atomics
// (self-contained, so no fences are needed). It moves from "empty" (all ones, set by a small fill
// kernel before each launch, which also zeroes the tickets) to the aggregate (A, U) to the
// inclusive state (a NaN tag in the low half, h in the high half); one lane writes both, so a
// reader never sees them out of order.
// Because the look-back combines whatever predecessors have published so far, the association
// order of the carry (not the math) depends on timing: results are reproducible to the fp32
// rounding of the carried state, not bit for bit.
#include <algorithm>

#include "rglru_launch.h"
#include "rglru_mfma.h"

namespace rglru {

constexpr int kFusedRows = 64;
constexpr unsigned kWaitVm0 = 0x0F70;     // s_waitcnt operand: vmcnt(0) only

typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }
constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor word 3: raw 32-bit data, no swizzle

// A workgroup owns one head for its whole life (persistent) and walks that head's tiles in
// ticket order: one wave per 32 channels (8 waves for Dh = 256, two per SIMD, one workgroup per
// CU with a 100 KB LDS tile pair). Each wave keeps its channels' W_a / W_x rows -- the MFMA B
// operand, 128 VGPRs at Dh = 256 -- in registers for the whole kernel, so the tile loop touches
// HBM only for x and y. The conv of a tile is computed once, for all Dh channels.
template <int DH> struct Fused {
  static constexpr int kNW = DH / 32;                // waves, 32 channels each
  static constexpr int kThreads = 64 * kNW;
  static constexpr int kKS = DH / 16;                // MFMA k-steps
  static constexpr int kLda = DH + 8;                // bf16 A-tile row stride (elements)
  static constexpr int kLdx = DH + 2;  // fp32 conv-output row stride: rows 16 apart 32 banks apart
  static constexpr int kRowsPerLoad = 1024 / (2 * DH);  // x rows per wave-wide 16 B/lane load
  static constexpr int kLoads = (kFusedRows + 3 + kRowsPerLoad - 1) / kRowsPerLoad;
  static constexpr int kXRows = kLoads * kRowsPerLoad;  // staged rows (tile + 3-row halo)
};


__device__ __forceinline__ bf16x8_t f32x8_to_bf16x8(const float *p) {
  const float4 v0 = *reinterpret_cast<const float4 *>(p);
  const float4 v1 = *reinterpret_cast<const float4 *>(p + 4);
  u32x4_t u;
  u[0] = pack_bf16x2(v0.x, v0.y);
  u[1] = pack_bf16x2(v0.z, v0.w);
  u[2] = pack_bf16x2(v1.x, v1.y);
  u[3] = pack_bf16x2(v1.z, v1.w);
  return __builtin_bit_cast(bf16x8_t, u);
}

// Look-back words to kEmpty and control words to 0: [0] unused, [1] count of lanes that gave up
// waiting, [2 + g] the tile ticket of head g.
// (extra: one more word to 0, or NULL -- the failure count of a workspace whose control block
// lies elsewhere)
__global__ void fused_reset(unsigned long long *slots, size_t n, unsigned *ctrl, int nctrl,
                            unsigned *extra) {
  fill_lookback(slots, n, ctrl, nctrl);
  if (extra && blockIdx.x == 0 && threadIdx.x == 0) *extra = 0u;
}

__global__ void clear_words(unsigned *p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

hipError_t launch_clear_words(unsigned *p, int n, hipStream_t s) {
  clear_words<<<1, 64, 0, s>>>(p, n);
  return hipGetLastError();
}

struct TileCtx {
  int j, tt, b, t0;
};

// Stage the x rows t0-3 .. t0+63 of one (sequence, head) tile -- the tile plus the conv halo --
// into LDS with direct buffer-to-LDS loads (16 bytes per lane, one contiguous 1 KB block per
// load), spread over the waves. They go through dma_16b, which the compiler does not track (for
// the builtin it cannot tell which LDS bytes the loads write, and would make the first LDS read
// after them -- the gate math's -- wait for all of them); the kernel waits for them itself
// (vmcnt) before the barrier that hands the rows to the conv. The buffer covers exactly sequence b, so its range check returns
// zeros for rows before t = 0 (the causal zero padding; negative offsets wrap past the end) and
// for rows past T-1 (which only feed rows that are not stored).
template <int DH, int NW>
__device__ __forceinline__ void stage_x(const bf16_t *__restrict__ x, bf16_t *xr, int b, int t0,
                                        int g, int w, int lane, int T, int D) {
  typedef Fused<DH> F;
  constexpr int kLanesPerRow = DH / 8;
  constexpr int kPerWave = (F::kLoads + NW - 1) / NW;
  const __amdgpu_buffer_rsrc_t seq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(x + static_cast<size_t>(b) * T * D), static_cast<short>(0),
      rec_bytes(T, D, 2u), kBufferWord3);
  // opaque: keeps the compiler from folding the lane's row into a 64-bit multiply-add per load
  unsigned lane_off =
      static_cast<unsigned>((lane / kLanesPerRow) * 2 * D + g * DH * 2 + (lane % kLanesPerRow) * 16);
  asm volatile("" : "+v"(lane_off));
  const unsigned base = lds_addr(xr);
#pragma unroll
  for (int k = 0; k < kPerWave; ++k) {
    const int i = w + k * NW;  // wave-uniform
    if (kPerWave * NW == F::kLoads || i < F::kLoads) {
      const unsigned row_off = row_bytes(t0 - 3 + i * F::kRowsPerLoad, D, 2u);
      dma_16b(seq, row_off + lane_off, base + i * F::kRowsPerLoad * DH * 2u);
    }
  }
}

// Conv prologue of one tile, fp32, from the staged rows (LDS row k holds time t0 - 3 + k, zero
// before t = 0) into xa (bf16, the MFMA A operand) and xf (fp32, for the input term). Thread role:
// channel pair pc0/pc0+1, rows pr0 .. pr0+PRPG-1. The role is re-derived from an opaque copy of
// the thread index on every call so that none of it stays live (and gets spilled) across the
// rest of the tile. A wave spans whole row groups only when a row group is >= 64 lanes wide
// (Dh >= 128); then the row index is wave-uniform and stays scalar.
template <int DH, bool WITH_XA = true>
__device__ __forceinline__ void conv_prologue(const bf16_t *xr, bf16_t *xa, float *xf,
                                              const uint32_t *cws, int tid) {
  typedef Fused<DH> F;
  constexpr int PP = DH / 2;
  constexpr int PRPG = kFusedRows * PP / F::kThreads;
  constexpr int PSUB = PRPG > 4 ? 4 : PRPG;  // rows per batch (bounds live registers)
  int tidv = tid;
  asm volatile("" : "+v"(tidv));
  const int pc0 = 2 * (tidv % PP);
  const int pr0 = PP % 64 == 0 ? __builtin_amdgcn_readfirstlane((tidv / PP) * PRPG)
                               : (tidv / PP) * PRPG;
  // Words hold a bf16 pair of the two channels (taps: cws[k] = w_k of both). The conv output
  // w0 x_{t-3} + w1 x_{t-2} + w2 x_{t-1} + w3 x_t is two bf16 dot products per channel (the
  // products are exact in fp32), on time pairs (x_k, x_{k+1}) of one channel gathered with a
  // byte permute.
  uint32_t cw[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) cw[k] = cws[k * PP + (pc0 >> 1)];
  constexpr uint32_t kLoPair = 0x05040100u, kHiPair = 0x07060302u;  // low / high halves of 2 words
  const bf16x2_t w01l = as_bf16x2(__builtin_amdgcn_perm(cw[1], cw[0], kLoPair));
  const bf16x2_t w23l = as_bf16x2(__builtin_amdgcn_perm(cw[3], cw[2], kLoPair));
  const bf16x2_t w01h = as_bf16x2(__builtin_amdgcn_perm(cw[1], cw[0], kHiPair));
  const bf16x2_t w23h = as_bf16x2(__builtin_amdgcn_perm(cw[3], cw[2], kHiPair));
#pragma unroll
  for (int rb = 0; rb < PRPG; rb += PSUB) {
    uint32_t xv[PSUB + 3];
#pragma unroll
    for (int k = 0; k < PSUB + 3; ++k)
      xv[k] = *reinterpret_cast<const uint32_t *>(xr + (pr0 + rb + k) * DH + pc0);
    bf16x2_t pl[PSUB + 2], ph[PSUB + 2];  // (x_k, x_{k+1}) of the low / high channel
#pragma unroll
    for (int k = 0; k < PSUB + 2; ++k) {
      pl[k] = as_bf16x2(__builtin_amdgcn_perm(xv[k + 1], xv[k], kLoPair));
      ph[k] = as_bf16x2(__builtin_amdgcn_perm(xv[k + 1], xv[k], kHiPair));
    }
#pragma unroll
    for (int r = 0; r < PSUB; ++r) {
      const float o0 = __builtin_amdgcn_fdot2_f32_bf16(
          pl[r + 2], w23l, __builtin_amdgcn_fdot2_f32_bf16(pl[r], w01l, 0.0f, false), false);
      const float o1 = __builtin_amdgcn_fdot2_f32_bf16(
          ph[r + 2], w23h, __builtin_amdgcn_fdot2_f32_bf16(ph[r], w01h, 0.0f, false), false);
      const int row = pr0 + rb + r;
      if (WITH_XA) *reinterpret_cast<uint32_t *>(xa + row * F::kLda + pc0) = pack_bf16x2(o0, o1);
      *reinterpret_cast<float2 *>(xf + row * F::kLdx + pc0) = make_float2(o0, o1);
    }
  }
}

// The gate math of one element in two steps, with the wave-uniform expm1 doubling (below)
// between them for the whole run (a branch per element would split every step into its own
// block and keep the scheduler from overlapping neighbouring elements).
// Step (a): r = sigmoid(pa) with exp2(-log2(e) (pa + b_a)) (ba2 = -log2(e) b_a folded into one
// FMA), then e' = expm1(kd r 2^-nh) by the polynomial.
__device__ __forceinline__ float gate_a(float pa, float kds, float ba2) {
  const float r = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(fmaf(pa, -kLog2e, ba2)));
  return expm1_poly(kds * r);
}
// e = expm1(log a) from e' by nh exact doublings e <- e (e + 2) (nh is wave-uniform, 0 unless the
// wave holds a channel with a^c < e^-1/4), over n accumulators of one run.
__device__ __forceinline__ void gate_double(f32x16_t &e, int lo, int n, int nh) {
  if (nh > 0) {
    for (int i = 0; i < nh; ++i)
#pragma unroll
      for (int jj = lo; jj < lo + n; ++jj) e[jj] *= e[jj] + 2.0f;
    // a = exp(log a) >= 0: clamp what rounding may leave below -1
#pragma unroll
    for (int jj = lo; jj < lo + n; ++jj) e[jj] = fmaxf(e[jj], -1.0f);
  }
}
// Step (b): a = 1 + e, m = sqrt(1 - a^2) = sqrt(-e (2 + e)), i = sigmoid(px), u = m i x; then the
// run's product and state advance, P <- P a, S <- a S + u (from P = 1, S = 0 at the run's start);
// the caller overwrites the accumulators with (P, S).
__device__ __forceinline__ void gate_b(float e, float px, float xv, float bx2, float &P, float &S,
                                       bool first) {
  const float a = 1.0f + e;
  const float m = __builtin_amdgcn_sqrtf(-e * (2.0f + e));
  const float ig =
      __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(fmaf(px, -kLog2e, bx2)));
  const float u = m * (ig * xv);
  S = first ? u : fmaf(a, S, u);
  P = first ? a : P * a;
}

// One tile per loop iteration:
//   [barrier] claim k+1 | conv(k) from the staged rows | [barrier] MFMA(k) | publish k+1 and stage
//   its rows | gates + scan(k) | look-back(k) | wait for the staged rows | fix-up and store y(k).
// Rows past the end of the sequence (only in the last tile) are computed like the others from
// zero input -- they come after every real row, so they cannot change a real row's state -- and
// only their stores are masked; h_T is then taken at row T-1 instead of at the end of the tile.
//
// PRE: the split plan's scan. The gate pre-activations (biases included) come from pre, fp16
// pairs (pa, px) [B][T][D] written by the gate kernel, instead of the MFMAs: each lane loads its
// 32 elements straight into the accumulator layout (a half-wave reads one 128-byte line per
// row), one tile ahead. Without the resident weights the registers hold both tiles. The next
// tile's ticket is then published before the conv barrier, so that every wave can issue those
// loads after it. Everything else -- conv for the input term, gates, scan, look-back, fix-up --
// is the same code.
template <int DH, bool PRE>
__global__ __launch_bounds__(Fused<DH>::kThreads, 2) void fused_forward(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ conv_w,
    const bf16_t *__restrict__ W_a, const float *__restrict__ b_a,
    const bf16_t *__restrict__ W_x, const float *__restrict__ b_x,
    const uint32_t *__restrict__ pre,
    const float *__restrict__ Lambda, const float *__restrict__ h0, bf16_t *__restrict__ y,
    float *__restrict__ h_T, int B, int T, int D, int H, int nTT, unsigned *ctrl,
    unsigned *gave_up, unsigned long long *slots) {
  typedef Fused<DH> F;
  constexpr int PP = DH / 2;  // channel pairs
  // xa: the conv output in bf16, the MFMA A operand; xf: the same in fp32 for the input term;
  // xr: the staged x rows.
  __shared__ __attribute__((aligned(16))) bf16_t xa[PRE ? 8 : kFusedRows * F::kLda];
  __shared__ __attribute__((aligned(16))) float xf[kFusedRows * F::kLdx];
  __shared__ __attribute__((aligned(16))) bf16_t xr[F::kXRows * DH];
  __shared__ uint32_t cws[4 * PP];  // conv taps of the head, bf16 pairs
  __shared__ int s_tile[3];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lrow = lane & 31;
  const int half = lane >> 5;
  const int g = blockIdx.x % H;
  const int ntiles = B * nTT;
  unsigned *ticket = ctrl + 2 + g;
  const int cl = w * 32 + lrow;  // this lane's channel within the head
  const int d = g * DH + cl;
  const float kd = decay_coeff(Lambda[d]);
  const float ba2 = PRE ? 0.0f : -kLog2e * b_a[d], bx2 = PRE ? 0.0f : -kLog2e * b_x[d];
  // B operand of this wave: its 32 channels' W_a / W_x rows, resident for the kernel's life
  bf16x8_t wa[F::kKS], wx[F::kKS];
  if (!PRE) {
    const bf16_t *wa_row = W_a + (static_cast<size_t>(g) * DH + cl) * DH + half * 8;
    const bf16_t *wx_row = W_x + (static_cast<size_t>(g) * DH + cl) * DH + half * 8;
#pragma unroll
    for (int ks = 0; ks < F::kKS; ++ks) {
      wa[ks] = load_bf16x8(wa_row + ks * 16);
      wx[ks] = load_bf16x8(wx_row + ks * 16);
    }
  }
  // kThreads == 4 * PP: one tap pair per thread
  cws[tid] = *reinterpret_cast<const uint32_t *>(conv_w + static_cast<size_t>(tid / PP) * D +
                                                 g * DH + 2 * (tid % PP));
  // log a = kd r >= kd: halve until every channel of the wave is inside the polynomial's range
  // (capped: beyond 2^-40, |kd| > 2.7e11 and a = 0 to fp32 precision; the clamp then gives it)
  int nh = 0;
  while (nh < 40 && __any(kd * __builtin_ldexpf(1.0f, -nh) < -0.25f)) ++nh;
  nh = __builtin_amdgcn_readfirstlane(nh);
  const float kds = kd * __builtin_ldexpf(1.0f, -nh);

  // Tickets run one tile ahead: tile k+1 is claimed at the start of tile k, and after the MFMA
  // wave 0 publishes it and stages its rows, so the ticket round trip and the x loads overlap
  // the conv, the MFMA and the gate math. (Claiming further ahead lets a tile wait behind two
  // of its owner's tiles, and its successors in time wait on it.) s_tile is a ring of three.
  // PRE: this lane's 32 pre-activation pairs of tile j (time row 32 rt + 16 half + jj, channel
  // cl; rows past T read row T - 1: they only feed rows that are not stored)
  // The loads go through a buffer descriptor over sequence b's pre-activations: the row's byte
  // offset is wave-uniform and the lane's (channel, 16-row half) offset fixed, so each load costs
  // one 32-bit add (a clamped 64-bit index product was four VALU instructions per load); rows
  // past T read zeros from the range check (they only feed rows that are not stored).
  uint32_t pn[32];
  const unsigned pre_lane = (static_cast<unsigned>(d) + 16u * half * static_cast<unsigned>(D)) * 4u;
  auto load_pre = [&](int j) {
    const int b = j % B, t0 = (j / B) * kFusedRows;
    const __amdgpu_buffer_rsrc_t seq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t *>(pre + static_cast<size_t>(b) * T * D), static_cast<short>(0),
        rec_bytes(T, D, 4u), kBufferWord3);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj)
        pn[16 * rt + jj] = __builtin_amdgcn_raw_buffer_load_b32(
            seq, row_bytes(t0 + 32 * rt + jj, D, 4u) + pre_lane, 0, 0);
  };
  if (tid == 0) s_tile[0] = static_cast<int>(atomicAdd(ticket, 1u));
  __syncthreads();
  {
    const int j0 = __builtin_amdgcn_readfirstlane(s_tile[0]);
    if (j0 < ntiles) stage_x<DH, F::kNW>(x, xr, j0 % B, (j0 / B) * kFusedRows, g, w, lane, T, D);
    if (PRE && j0 < ntiles) load_pre(j0);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
  }

  int slot = 0;  // it % 3
  for (;;) {
    __syncthreads();  // this tile's conv in xa / xf; staging buffer free; tickets visible
    TileCtx tc;
    tc.j = __builtin_amdgcn_readfirstlane(s_tile[slot]);
    if (tc.j >= ntiles) break;
    const int slot1 = slot == 2 ? 0 : slot + 1;
    unsigned claim = 0;
    if (tid == 0) claim = atomicAdd(ticket, 1u);
    tc.tt = tc.j / B;
    tc.b = tc.j % B;
    tc.t0 = tc.tt * kFusedRows;
    conv_prologue<DH, !PRE>(xr, xa, xf, cws, tid);
    if (PRE && tid == 0) s_tile[slot1] = static_cast<int>(claim);
    __syncthreads();

    // ---- gate projections on MFMA: 64 rows x (32 channels x 2 gates) per wave. The A operand's
    // rows are permuted so that accumulator jj of lane (j, half) holds time row
    // rt*32 + 16*half + jj: every lane owns two runs of 16 consecutive steps of its channel.
    // Row tile 0 first; row tile 1's MFMAs are then interleaved, one k-step at a time, with the
    // gate math and scan of row tile 0 (one step per k-step), so that the matrix cores and the
    // vector ALU work at the same time.
    const int prow = 16 * ((lrow >> 2) & 1) + 4 * (lrow >> 3) + (lrow & 3);
    const bf16_t *xap = xa + prow * F::kLda + half * 8;
    f32x16_t acc[2][2];  // [row tile][gate]
    if constexpr (PRE) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          acc[rt][0][jj] = f16lo(pn[16 * rt + jj]);
          acc[rt][1][jj] = f16hi(pn[16 * rt + jj]);
        }
      // the next tile's pre-activations and x rows, in flight during this tile
      const int jn = __builtin_amdgcn_readfirstlane(s_tile[slot1]);
      if (jn < ntiles) {
        load_pre(jn);
        if (w == 0) stage_x<DH, 1>(x, xr, jn % B, (jn / B) * kFusedRows, g, 0, lane, T, D);
      }
    } else {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        acc[rt][0] = f32x16_t{};
        acc[rt][1] = f32x16_t{};
      }
#pragma unroll
      for (int ks = 0; ks < F::kKS; ++ks) {
        const bf16x8_t af = load_bf16x8(xap + ks * 16);
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, wa[ks], acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, wx[ks], acc[0][1], 0, 0, 0);
      }

      // ---- stage the next tile's rows (the prologue that read the buffer finished before the
      // barrier above); they land during the gate math.
      if (w == 0) {
        const int jn = __builtin_amdgcn_readfirstlane(claim);
        if (lane == 0) s_tile[slot1] = jn;
        if (jn < ntiles) stage_x<DH, 1>(x, xr, jn % B, (jn / B) * kFusedRows, g, 0, lane, T, D);
      }
    }

    // x of this lane's runs, fp32 (time row rt*32 + 16*half + jj, channel cl)
    const float *xfl = xf + 16 * half * F::kLdx + cl;
    float Ar[2], Ur[2];
    {
      // Row tile 1's k-steps carry row tile 0's gate math: step (a) of two elements per k-step
      // over the first half, the doublings, then step (b) and the scan of two elements per
      // k-step (Dh < 256: the MFMAs end early); x is read one k-step ahead.
      float P = 1.0f, S = 0.0f;
      float xn0 = xfl[0], xn1 = xfl[F::kLdx];
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        if (!PRE && ks < F::kKS) {
          const bf16x8_t af = load_bf16x8(xap + 32 * F::kLda + ks * 16);
          acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, wa[ks], acc[1][0], 0, 0, 0);
          acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, wx[ks], acc[1][1], 0, 0, 0);
        }
        if (ks < 8) {
          acc[0][0][2 * ks] = gate_a(acc[0][0][2 * ks], kds, ba2);
          acc[0][0][2 * ks + 1] = gate_a(acc[0][0][2 * ks + 1], kds, ba2);
        } else {
          const int jj = 2 * (ks - 8);
          if (ks == 8) gate_double(acc[0][0], 0, 16, nh);
          const float xv0 = xn0, xv1 = xn1;
          if (jj + 2 < 16) {
            xn0 = xfl[(jj + 2) * F::kLdx];
            xn1 = xfl[(jj + 3) * F::kLdx];
          }
          gate_b(acc[0][0][jj], acc[0][1][jj], xv0, bx2, P, S, jj == 0);
          acc[0][0][jj] = P;
          acc[0][1][jj] = S;
          gate_b(acc[0][0][jj + 1], acc[0][1][jj + 1], xv1, bx2, P, S, false);
          acc[0][0][jj + 1] = P;
          acc[0][1][jj + 1] = S;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      Ar[0] = P;
      Ur[0] = S;
    }
    {
      // row tile 1: step (a), the doublings, step (b) and the scan
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        acc[1][0][jj] = gate_a(acc[1][0][jj], kds, ba2);
        if ((jj & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
      gate_double(acc[1][0], 0, 16, nh);
      float P = 1.0f, S = 0.0f;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        gate_b(acc[1][0][jj], acc[1][1][jj], xfl[(32 + jj) * F::kLdx], bx2, P, S, jj == 0);
        acc[1][0][jj] = P;
        acc[1][1][jj] = S;
        if ((jj & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
      Ar[1] = P;
      Ur[1] = S;
    }
    // Runs in time order: (row tile 0, half 0), (0, 1), (1, 0), (1, 1). Every lane gets all
    // four maps and chains them: (q, c) = the start of one of its runs as an affine map of the
    // tile's carry-in; (At, Ut) = the whole tile.
    float A0, A1, A2, A3, U0, U1, U2, U3;
    halves(Ar[0], A0, A1);
    halves(Ar[1], A2, A3);
    halves(Ur[0], U0, U1);
    halves(Ur[1], U2, U3);
    const float q2 = A1 * A0, c2 = fmaf(A1, U0, U1);
    const float q3 = A2 * q2, c3 = fmaf(A2, c2, U2);
    const float At = A3 * q3, Ut = fmaf(A3, c3, U3);
    const float qa = half ? A0 : 1.0f, ca = half ? U0 : 0.0f;
    const float qb = half ? q3 : q2, cb = half ? c3 : c2;

    // ---- decoupled look-back on half 0 (one channel per lane): publish this tile's aggregate
    // and put the first predecessor's word in flight...
    const size_t slot_me = (static_cast<size_t>(tc.j) * H + g) * DH + cl;  // j = tt*B + b
    unsigned long long v = kEmpty;
    if (half == 0) {
      if (tc.tt + 1 < nTT) st_relaxed(slots + slot_me, pack2(At, Ut));
      if (tc.tt > 0)
        v = ld_relaxed(slots + ((static_cast<size_t>(tc.tt - 1) * B + tc.b) * H + g) * DH + cl);
    }

    // ... and finish the look-back: combine aggregates until an inclusive state (or the start
    // of the sequence) is found, then publish this tile's inclusive state.
    float h_in = 0.0f;
    if (half == 0) {
      const float *h0b = h0 ? h0 + static_cast<size_t>(tc.b) * D + d : nullptr;
      if (tc.tt == 0) {
        h_in = h0b ? *h0b : 0.0f;
      } else {
        float Aacc = 1.0f, Uacc = 0.0f;
        int jt = tc.tt - 1;
        unsigned spins = 0;
        for (;;) {
          if (is_incl(v)) {
            h_in = fmaf(Aacc, hi_f(v), Uacc);
            break;
          }
          if (v != kEmpty) {
            Uacc = fmaf(Aacc, hi_f(v), Uacc);
            Aacc *= lo_f(v);
            if (--jt < 0) {
              h_in = fmaf(Aacc, h0b ? *h0b : 0.0f, Uacc);
              break;
            }
          } else {
            if (++spins > kMaxSpin) {
              atomicAdd(gave_up, 1u);
              h_in = __builtin_nanf("");
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
          v = ld_relaxed(slots + ((static_cast<size_t>(jt) * B + tc.b) * H + g) * DH + cl);
        }
      }
      const float h_end = fmaf(At, h_in, Ut);
      if (tc.tt + 1 < nTT)
        st_relaxed(slots + slot_me, pack_incl(h_end));
      else if (h_T && tc.t0 + kFusedRows == T)
        h_T[static_cast<size_t>(tc.b) * D + d] = h_end;
    }
    {
      float hl, hh;
      halves(h_in, hl, hh);
      h_in = hl;
    }
    // The staged rows must have landed before the barrier that opens the next tile; waiting here
    // (the look-back has mostly waited already) keeps this tile's stores out of the wait.
    __builtin_amdgcn_s_waitcnt(kWaitVm0);

    // ---- fix-up h_t = P_t * (state at its run's start) + S_t and store y, two rows per bf16
    // conversion, the halves stored separately. Row addresses are wave-uniform: a scalar row
    // pointer plus the lane's 32-bit byte offset (its channel and its half's 16-row shift). Dv is
    // re-materialised
    // through an empty asm so that the compiler cannot hoist the 32 row offsets out of the tile
    // loop (it would keep them in registers, spill them and reload one per store).
    unsigned Dv = static_cast<unsigned>(D);
    asm volatile("" : "+s"(Dv));
    const char *yg = reinterpret_cast<const char *>(
        y + (static_cast<size_t>(tc.b) * T + tc.t0) * D + g * DH);  // tile row 0, head g
    const unsigned lane_off = (static_cast<unsigned>(cl) + 16u * half * Dv) * 2u;
    const float carry[2] = {fmaf(qa, h_in, ca), fmaf(qb, h_in, cb)};
    if (tc.t0 + kFusedRows <= T) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int jj = 0; jj < 16; jj += 2) {
          uint32_t pk = pack_bf16x2(fmaf(acc[rt][0][jj], carry[rt], acc[rt][1][jj]),
                                    fmaf(acc[rt][0][jj + 1], carry[rt], acc[rt][1][jj + 1]));
          asm volatile("" : "+v"(pk));  // keep one conversion for the pair
          char *row0 = const_cast<char *>(yg) + (rt * 32 + jj) * Dv * 2u;
          *reinterpret_cast<bf16_t *>(row0 + lane_off) = static_cast<bf16_t>(pk);
          *reinterpret_cast<bf16_t *>(row0 + Dv * 2u + lane_off) = static_cast<bf16_t>(pk >> 16);
        }
    } else {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const float hv = fmaf(acc[rt][0][jj], carry[rt], acc[rt][1][jj]);
          const int t = tc.t0 + rt * 32 + 16 * half + jj;
          char *row0 = const_cast<char *>(yg) + (rt * 32 + jj) * Dv * 2u;
          if (t < T) *reinterpret_cast<bf16_t *>(row0 + lane_off) = f32_to_bf16(hv);
          if (t == T - 1 && h_T) h_T[static_cast<size_t>(tc.b) * D + d] = hv;
        }
    }
    slot = slot1;
  }
}

size_t fused_ctrl_bytes(int H) { return (static_cast<size_t>(2 + H) * 4 + 255) / 256 * 256; }

size_t fused_slots(int B, int T, int H, int Dh) {
  const size_t nTT = (T + kFusedRows - 1) / kFusedRows;
  return nTT * B * H * Dh;
}

bool fused_supported(int io, int T, int D, int Dh) {
  // byte offsets within one sequence, halo included, stay below 2^32 and wrap past its end
  return io == kBF16 && (Dh == 32 || Dh == 64 || Dh == 128 || Dh == 256) &&
         (static_cast<long long>(T) + 3) * D < (1LL << 31);
}

hipError_t launch_fused(const void *x, const void *conv_w, const void *W_a, const float *b_a,
                        const void *W_x, const float *b_x, const float *Lambda, const float *h0,
                        void *y, float *h_T, int B, int T, int D, int H, void *ctrl_ws,
                        hipStream_t s) {
  const int Dh = D / H;
  const int nTT = (T + kFusedRows - 1) / kFusedRows;
  const size_t nslot = fused_slots(B, T, H, Dh);
  unsigned *ctrl = static_cast<unsigned *>(ctrl_ws);
  unsigned long long *slots =
      reinterpret_cast<unsigned long long *>(static_cast<char *>(ctrl_ws) + fused_ctrl_bytes(H));
  fused_reset<<<fill_blocks(nslot), 256, 0, s>>>(slots, nslot, ctrl, 2 + H, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const bf16_t *xx = static_cast<const bf16_t *>(x);
  const bf16_t *cw = static_cast<const bf16_t *>(conv_w);
  const bf16_t *wa = static_cast<const bf16_t *>(W_a);
  const bf16_t *wx = static_cast<const bf16_t *>(W_x);
  bf16_t *yy = static_cast<bf16_t *>(y);
  // Persistent grid: about one workgroup per CU, the same number for every head. Extra
  // workgroups that only start once others exit find the tickets used up and leave.
#define RGLRU_FUSED_CASE(DHV)                                                                   \
  case DHV: {                                                                                   \
    const int per = std::max(1, (cus + H - 1) / H);                                             \
    fused_forward<DHV, false><<<H * per, Fused<DHV>::kThreads, 0, s>>>(                         \
        xx, cw, wa, b_a, wx, b_x, nullptr, Lambda, h0, yy, h_T, B, T, D, H, nTT, ctrl, ctrl + 1, \
        slots);                                                                                 \
    break;                                                                                      \
  }
  switch (Dh) {
    RGLRU_FUSED_CASE(32)
    RGLRU_FUSED_CASE(64)
    RGLRU_FUSED_CASE(128)
    RGLRU_FUSED_CASE(256)
    default: return hipErrorInvalidValue;
  }
#undef RGLRU_FUSED_CASE
  return hipGetLastError();
}

// Channel groups of the split plan's scan. Without the gate contraction nothing ties a
// workgroup to a whole head: every channel's recurrence is independent once its
// pre-activations are given. Heads of 256 channels are therefore scanned as groups of 128 (four
// waves, 52 KB of LDS), several workgroups per CU that share no barrier, so one's look-back or
// stores overlap another's gate math.
int scan_tiled_group(int Dh) { return Dh == 256 ? 128 : Dh; }
int scan_tiled_groups(int D, int H) { return D / scan_tiled_group(D / H); }
// Workgroups of the scan per CU (grid = this many per CU's worth of groups; they are resident
// together at Dh 128: 167 VGPRs allow three waves per SIMD, the LDS three workgroups).
static int scan_tiled_per_cu(int G) { return G == 128 ? 3 : 1; }

// The split plan's scan over 64-step tiles chained by the same look-back (bf16, Dh in
// {32, 64, 128, 256}): pre holds the gate pre-activations (fp16 pairs, biases included); ctrl:
// 2 + scan_tiled_groups(D, H) words (tickets), words: fused_slots(B, T, H, Dh) look-back words
// (the same count under any grouping), both reset here; gave_up: the count of lanes whose
// look-back wait gave up (reset here too).
hipError_t launch_scan_tiled(const void *x, const void *pre, const void *conv_w,
                             const float *Lambda, const float *h0, void *y, float *h_T, int B,
                             int T, int D, int H, unsigned *ctrl, unsigned *gave_up,
                             unsigned long long *words, hipStream_t s) {
  const int G = scan_tiled_group(D / H);  // channels per workgroup
  const int Hg = D / G;                   // channel groups, each scanned like a head
  const int nTT = (T + kFusedRows - 1) / kFusedRows;
  const size_t nslot = fused_slots(B, T, Hg, G);
  fused_reset<<<fill_blocks(nslot), 256, 0, s>>>(words, nslot, ctrl, 2 + Hg,
                                                 gave_up == ctrl + 1 ? nullptr : gave_up);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const bf16_t *xx = static_cast<const bf16_t *>(x);
  const bf16_t *cw = static_cast<const bf16_t *>(conv_w);
  const uint32_t *pp = static_cast<const uint32_t *>(pre);
  bf16_t *yy = static_cast<bf16_t *>(y);
#define RGLRU_TILED_CASE(DHV)                                                                   \
  case DHV: {                                                                                   \
    const int per = std::max(1, (scan_tiled_per_cu(G) * cus + Hg - 1) / Hg);                   \
    fused_forward<DHV, true><<<Hg * per, Fused<DHV>::kThreads, 0, s>>>(                         \
        xx, cw, nullptr, nullptr, nullptr, nullptr, pp, Lambda, h0, yy, h_T, B, T, D, Hg, nTT,   \
        ctrl, gave_up, words);                                                                  \
    break;                                                                                      \
  }
  switch (G) {
    RGLRU_TILED_CASE(32)
    RGLRU_TILED_CASE(64)
    RGLRU_TILED_CASE(128)
    RGLRU_TILED_CASE(256)
    default: return hipErrorInvalidValue;
  }
#undef RGLRU_TILED_CASE
  return hipGetLastError();
}

}  // namespace rglru
