// rglru_bwd_fused.hip -- the backward's per-element part in one pass over 32-step tiles (bf16,
// Dh in {128, 256}): the gate pre-activations recomputed from x, the adjoint recurrence run
// backward in time, and the per-element gradients, without writing the pre-activations or the
// chunk maps to HBM.
//
// Per (b, d) and time t (the notation of rglru_backward.hip, which holds the derivation):
//   delta_t = dy_t + g_{t+1},  g_t = a_t delta_t,  g at the end of the sequence = dh_T,  dh0 = g_0,
// and from delta the gradients dpa, dpx, the direct part of dxc, and per-tile partial sums of dpa,
// dpx and r dz. Over one tile, g_start = A g_end + U (A = product of a over the tile, U = g_start
// when g_end = 0): an affine map, so tiles are chained like the forward's fused plan, backward in
// time.
//
// A workgroup owns one head for its whole life (persistent) and takes that head's tiles by
// ticket, latest time first (ticket j: sequence j % B, tile nTT - 1 - j / B). Per tile:
//   conv of the staged x rows (fp32 dot products of bf16 pairs) into bf16 hi + lo | the next
//   tile's x, dy and y rows staged by direct buffer-to-LDS loads (the lane phase reads all three
//   from LDS: per-lane global loads there waited on memory at two waves per SIMD; 32-row tiles
//   keep the three double-buffered tiles inside the LDS) | [32 x Dh] x [Dh x 2Dh] on MFMA with the
//   head's W_a / W_x rows resident in registers (A = hi + lo, as in the separate pre-activation
//   kernel: the gradients amplify pre-activation errors through r (1 - r) and 1/m) | the
//   pre-activations as fp16 pairs into LDS over the conv tile | lane phase: thread = (channel
//   pair, 16-row segment); pass 1 walks the segment backward for its map (A, U) | the tile's
//   map, g at the tile's end from the next tile in time, g at its start published for the
//   previous tile | pass 2 walks the segment backward again from its own g and writes the
//   gradients.
// The carry is the fold of the later tiles' maps from dh_T, taken from the nearest published
// g_start and the maps in between, always in the fold's own order, so every result is the same
// bitwise from run to run. Maps are published before any wait, so a tile's wait ends as soon as
// the tiles after it have finished their first pass; it is bounded all the same (a lost word
// gives NaN and bumps a counter, never a hang).
#include <algorithm>
#include <type_traits>

#include "rglru_launch.h"
#include "rglru_mfma.h"

namespace rglru {

namespace {
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
constexpr int kRawWord3 = 0x00020000;  // buffer descriptor word 3: raw 32-bit data, no swizzle
constexpr uint32_t kLoPair = 0x05040100u, kHiPair = 0x07060302u;  // low / high 16-bit halves
constexpr int kRows = kFusedBwdRows;                               // rows per tile (32)
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }
}  // namespace

template <int DH> struct BwdTile {
  static_assert(DH == 128 || DH == 256, "fused backward tile needs Dh in {128, 256}");
  static constexpr int kNW = DH / 32;                // waves, 32 channels each for the MFMA
  static constexpr int kThreads = 64 * kNW;          // = 2 Dh
  static constexpr int kKS = DH / 16;                // MFMA k-steps
  static constexpr int kLda = DH + 8;                // bf16 A-tile row stride
  static constexpr int kRowsPerLoad = 1024 / (2 * DH);  // rows per wave-wide 16 B/lane load
  static constexpr int kXLoads = (kRows + 3 + kRowsPerLoad - 1) / kRowsPerLoad;
  static constexpr int kXRows = kXLoads * kRowsPerLoad;  // staged x rows: tile + 3-row halo
  static constexpr int kRLoads = kRows / kRowsPerLoad;   // dy (and y) loads per tile
  static constexpr int kLoads = kXLoads + 2 * kRLoads;
  static constexpr int kPP = DH / 2;                 // channel pairs (conv role)
  static constexpr int kCRows = kRows * kPP / kThreads;  // conv rows per thread (8)
  static constexpr int kSeg = kThreads / DH;         // row segments of the lane phase (2)
  static constexpr int kSegRows = kRows / kSeg;      // 16
  static_assert(kSeg == 2 && kRows * DH * 4 <= 2 * kRows * kLda * 2, "layout");
};

// dpre / dxc / part / dh0 as the separate per-element kernel writes them (layouts in
// rglru_backward.hip: dpre holds (dpa, dpx) as fp16 pairs); words: [nTT][B][D] (each tile's map
// (A, U), later g at its start), all kEmpty; ctrl: [1] give-up count, [2 + g] head g's ticket, all 0.
template <int DH>
__global__ __launch_bounds__(BwdTile<DH>::kThreads, 1) void tile_bwd(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ y, const bf16_t *__restrict__ dy,
    const float *__restrict__ h0, const float *__restrict__ dh_T, const bf16_t *__restrict__ conv_w,
    const bf16_t *__restrict__ W_a, const float *__restrict__ b_a, const bf16_t *__restrict__ W_x,
    const float *__restrict__ b_x, const float *__restrict__ Lambda, uint32_t *__restrict__ dpre,
    uint16_t *__restrict__ dxc, float *__restrict__ part,
    float *__restrict__ dh0, int B, int T, int D, int H, int nTT, unsigned *ctrl,
    unsigned long long *words) {
  typedef BwdTile<DH> F;
  __shared__ __attribute__((aligned(16))) bf16_t xr[2][F::kXRows * DH];  // x rows t0-3 ..
  __shared__ __attribute__((aligned(16))) bf16_t dyr[2][kRows * DH];     // dy rows t0 ..
  __shared__ __attribute__((aligned(16))) bf16_t yr[2][kRows * DH];      // y rows t0-1 ..
  __shared__ __attribute__((aligned(16))) bf16_t xa[2 * kRows * F::kLda];  // conv hi / lo
  __shared__ int s_tile[2];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lrow = lane & 31;
  const int half = lane >> 5;
  const int g = blockIdx.x % H;
  const int ntiles = B * nTT;
  unsigned *ticket = ctrl + 2 + g;
  // This lane's channel (the MFMA output column) and its W_a / W_x rows (the B operand). The lane
  // phase works on the accumulators where they are: lane (channel, half) holds tile rows
  // 16 half .. 16 half + 15 of its channel, because the A operand's rows are fed permuted (lane i
  // of the A operand supplies tile row 16 ((i / 4) mod 2) + 4 (i / 8) + i mod 4).
  const int cl = w * 32 + lrow;
  const int prow = 16 * ((lrow >> 2) & 1) + 4 * (lrow >> 3) + (lrow & 3);
  const float ba = b_a[g * DH + cl], bx = b_x[g * DH + cl];
  bf16x8_t wa[F::kKS], wx[F::kKS];
  {
    const bf16_t *ra = W_a + (static_cast<size_t>(g) * DH + cl) * DH + half * 8;
    const bf16_t *rx = W_x + (static_cast<size_t>(g) * DH + cl) * DH + half * 8;
#pragma unroll
    for (int ks = 0; ks < F::kKS; ++ks) {
      wa[ks] = load_bf16x8(ra + ks * 16);
      wx[ks] = load_bf16x8(rx + ks * 16);
    }
  }
  // conv role: channel pair cp (channels 2cp, 2cp + 1), tile rows cr * kCRows ..
  const int cp = tid % F::kPP;
  const int cr = tid / F::kPP;
  const int dc = g * DH + cl;
  // conv taps of the channel pair (conv role) as bf16 pairs (w0, w1), (w2, w3)
  bf16x2_t w01l, w23l, w01h, w23h;
  {
    uint32_t cw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      cw[k] = *reinterpret_cast<const uint32_t *>(conv_w + static_cast<size_t>(k) * D + g * DH + 2 * cp);
    w01l = as_bf16x2(__builtin_amdgcn_perm(cw[1], cw[0], kLoPair));
    w23l = as_bf16x2(__builtin_amdgcn_perm(cw[3], cw[2], kLoPair));
    w01h = as_bf16x2(__builtin_amdgcn_perm(cw[1], cw[0], kHiPair));
    w23h = as_bf16x2(__builtin_amdgcn_perm(cw[3], cw[2], kHiPair));
  }
  const float kd = decay_coeff(Lambda[dc]);
  // expm1(log a) takes the polynomial alone unless some channel of the wave has a decay below
  // e^-1/4 (log a can then leave the polynomial's range): a wave-uniform choice of loop variant,
  // so the usual decays never evaluate the exp2 of the other branch
  const bool fast = __builtin_amdgcn_readfirstlane(__any(kd < -0.25f) ? 1 : 0) != 0;

  // conv of staged rows q .. q+3 (time t - 3 .. t for tile row q), as pair words: both channels
  // of the pair
  auto conv2 = [&](const uint32_t (&xv)[4], float &o0, float &o1) {
    o0 = __builtin_amdgcn_fdot2_f32_bf16(
        as_bf16x2(__builtin_amdgcn_perm(xv[3], xv[2], kLoPair)), w23l,
        __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(__builtin_amdgcn_perm(xv[1], xv[0], kLoPair)), w01l,
                                        0.0f, false),
        false);
    o1 = __builtin_amdgcn_fdot2_f32_bf16(
        as_bf16x2(__builtin_amdgcn_perm(xv[3], xv[2], kHiPair)), w23h,
        __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(__builtin_amdgcn_perm(xv[1], xv[0], kHiPair)), w01h,
                                        0.0f, false),
        false);
  };
  // staging of tile j into buffer bf: x rows t0-3 .. t0+31 (+ a few unused), dy rows t0 ..
  // t0+31 and y rows t0-1 .. t0+30, spread over the waves. Each buffer covers exactly sequence
  // b, so its range check returns zeros before t = 0 (negative offsets wrap past the end) and
  // past T - 1.
  constexpr int kLanesPerRow = DH / 8;
  const unsigned lane_off =
      static_cast<unsigned>((lane / kLanesPerRow) * 2 * D + g * DH * 2 + (lane % kLanesPerRow) * 16);
  auto stage = [&](int j, int bf) {
    const int b = j % B, t0 = (nTT - 1 - j / B) * kRows;
    const size_t so = static_cast<size_t>(b) * T * D;
    const __amdgpu_buffer_rsrc_t sx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(x + so), static_cast<short>(0), rec_bytes(T, D, 2u),
        kRawWord3);
    const __amdgpu_buffer_rsrc_t sdy = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(dy + so), static_cast<short>(0), rec_bytes(T, D, 2u),
        kRawWord3);
    const __amdgpu_buffer_rsrc_t sy = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(y + so), static_cast<short>(0), rec_bytes(T, D, 2u),
        kRawWord3);
    for (int i = w; i < F::kLoads; i += F::kNW) {  // wave-uniform
      if (i < F::kXLoads) {
        const unsigned row_off = row_bytes(t0 - 3 + i * F::kRowsPerLoad, D, 2u);
        dma_16b(sx, row_off + lane_off, lds_addr(xr[bf] + i * F::kRowsPerLoad * DH));
      } else if (i < F::kXLoads + F::kRLoads) {
        const int q = i - F::kXLoads;
        const unsigned row_off = row_bytes(t0 + q * F::kRowsPerLoad, D, 2u);
        dma_16b(sdy, row_off + lane_off, lds_addr(dyr[bf] + q * F::kRowsPerLoad * DH));
      } else {
        const int q = i - F::kXLoads - F::kRLoads;
        const unsigned row_off = row_bytes(t0 - 1 + q * F::kRowsPerLoad, D, 2u);
        dma_16b(sy, row_off + lane_off, lds_addr(yr[bf] + q * F::kRowsPerLoad * DH));
      }
    }
  };

  if (tid == 0) s_tile[0] = static_cast<int>(atomicAdd(ticket, 1u));
  __syncthreads();
  {
    const int j0 = __builtin_amdgcn_readfirstlane(s_tile[0]);
    if (j0 < ntiles) stage(j0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): own staging loads landed
  }
  // Barriers inside the loop order LDS only (lds_barrier): the staging loads are waited for
  // explicitly (vmcnt(0) before pass 2, before the next tile's first barrier), and no global
  // memory is exchanged between the waves, so no barrier needs to wait for the gradient stores or
  // the staging loads in flight. After the MFMAs each wave works on its own channels alone.
  int cur = 0;
  for (;;) {
    lds_barrier();  // this tile's rows staged; the previous tile's LDS reads done
    const int j = __builtin_amdgcn_readfirstlane(s_tile[cur]);
    if (j >= ntiles) break;
    // The next ticket: its round trip overlaps the conv; written to LDS after it (vector memory
    // completes in issue order, so waiting for the ticket also waits for the previous tile's
    // gradient stores: the later the wait, the less of it is left).
    unsigned claim = 0;
    if (tid == 0) claim = atomicAdd(ticket, 1u);
    const int b = j % B, tt = nTT - 1 - j / B, t0 = tt * kRows;
    const bf16_t *xs = xr[cur];
    // The lane's roles again, from a thread index opaque to the compiler: otherwise it hoists
    // every per-lane address made from them (LDS rows, look-back words, h0, dh_T) out of the
    // loop and holds them in registers for the whole kernel, which does not fit next to the
    // resident weights. Rebuilding them costs a few instructions per tile.
    int tid_o = tid;
    asm volatile("" : "+v"(tid_o));
    const int lane = tid_o & 63, lrow = lane & 31, half = lane >> 5;
    const int cl = w * 32 + lrow, dc = g * DH + cl;
    const int cp = tid_o % F::kPP, cr = tid_o / F::kPP;
    const int prow = 16 * ((lrow >> 2) & 1) + 4 * (lrow >> 3) + (lrow & 3);
    // ---- conv -> hi / lo bf16
#pragma unroll 4
    for (int r = 0; r < F::kCRows; ++r) {
      const int row = cr * F::kCRows + r;  // staged row row + k holds time t0 - 3 + row + k
      uint32_t xv[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) xv[k] = *reinterpret_cast<const uint32_t *>(xs + (row + k) * DH + 2 * cp);
      float o0, o1;
      conv2(xv, o0, o1);
      const uint32_t hv = pack_bf16x2(o0, o1);
      *reinterpret_cast<uint32_t *>(xa + row * F::kLda + 2 * cp) = hv;
      *reinterpret_cast<uint32_t *>(xa + (kRows + row) * F::kLda + 2 * cp) =
          pack_bf16x2(o0 - bf16lo(hv), o1 - bf16hi(hv));
    }
    if (tid == 0) s_tile[cur ^ 1] = static_cast<int>(claim);
    lds_barrier();  // xa ready; the next ticket visible
    {
      const int jn = __builtin_amdgcn_readfirstlane(s_tile[cur ^ 1]);
      if (jn < ntiles) stage(jn, cur ^ 1);  // its last readers finished before the loop top
    }
    // ---- [32 x DH] x [DH x 2 DH]: A = hi + lo, rows permuted
    // (A operands loaded one k-step ahead, one k-step per scheduling region: the weights take
    // half the registers, so the loads must not all be in flight at once)
    f32x16_t acc[2];  // [gate]
    acc[0] = acc[1] = f32x16_t{};
    {
      const bf16_t *ap = xa + prow * F::kLda + half * 8;
      bf16x8_t af[2][2];  // [ks & 1][pt]
      af[0][0] = load_bf16x8(ap);
      af[0][1] = load_bf16x8(ap + kRows * F::kLda);
#pragma unroll
      for (int ks = 0; ks < F::kKS; ++ks) {
        if (ks + 1 < F::kKS) {
          af[(ks + 1) & 1][0] = load_bf16x8(ap + (ks + 1) * 16);
          af[(ks + 1) & 1][1] = load_bf16x8(ap + kRows * F::kLda + (ks + 1) * 16);
        }
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][pt], wa[ks], acc[0], 0, 0, 0);
          acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][pt], wx[ks], acc[1], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // ---- pass 1: this half's map g_start = A g_end + U over its 16 rows, walking them backward;
    // r (in place of its pre-activation) and expm1(log a) kept for pass 2. Rows at or past T
    // (only in the last tile) are the identity: a = 1, and dy there is 0 (the staging loads' range
    // check). Every load is unconditional, so the 16 rows are one block for the scheduler.
    const bf16_t *dyt = dyr[cur] + 16 * half * DH + cl;  // row jj: dy at t0 + 16 half + jj
    const bf16_t *yt = yr[cur] + 16 * half * DH + cl;    // row jj: y at t0 + 16 half + jj - 1
    const int tl = t0 + 16 * half;                        // time of this half's row 0
    float ev[16];
    float A = 1.0f, U = 0.0f;
    auto pass1 = [&](auto nh) {
      bf16_t dq[2];  // dy two rows ahead; each row fenced off for the scheduler
      dq[1] = dyt[15 * DH];
      dq[0] = dyt[14 * DH];
#pragma unroll
      for (int jj = 15; jj >= 0; --jj) {
        const float dyv = bf16_to_f32(dq[jj & 1]);
        if (jj >= 2) dq[jj & 1] = dyt[(jj - 2) * DH];
        const float rr = fast_sigmoid(acc[0][jj] + ba);
        const float z = kd * rr;
        const float ez = decltype(nh)::value ? expm1_nonpos(z) : expm1_poly(z);
        const float e = tl + jj < T ? ez : 0.0f;
        acc[0][jj] = rr;
        ev[jj] = e;
        const float a = 1.0f + e;
        U = a * (dyv + U);
        A *= a;
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (fast)
      pass1(std::true_type{});
    else
      pass1(std::false_type{});
    // ---- the tile's map, g at its end from the next tile in time, g at its start published
    // (half 0's lanes; g_start = A0 (A1 g_end + U1) + U0)
    float A0, A1, U0, U1;
    halves(A, A0, A1);
    halves(U, U0, U1);
    float gend = 0.0f;
    if (half == 0) {
      const float At = A1 * A0;
      const float Ut = fmaf(A0, U1, U0);
      // tile tt's word of this channel (word k at bd + k B D): empty, then its map (A, U), then
      // g at its start (tagged, in the high half)
      const size_t bd = static_cast<size_t>(b) * D + dc;
      const size_t tstride = static_cast<size_t>(B) * D;
      if (tt > 0) st_relaxed(words + bd + static_cast<size_t>(tt) * tstride, pack2(At, Ut));
      // g at the tile's end is the fold g <- A_k g + U_k over the later tiles k, from dh_T at the
      // sequence end. Find the nearest later tile whose g_start is out, passing tiles whose map is
      // out (a map never waits for anything), then fold back over the tiles in between in the
      // fold's own order, taking a tile's g_start where it is out by then and applying its map
      // otherwise: every g_start is an intermediate value of that one fold, so the result does
      // not depend on which words happened to be out (bitwise the same from run to run).
      int k = tt + 1;
      unsigned long long vi = kEmpty;
      unsigned spins = 0;
      bool lost = false;
      while (k < nTT) {
        vi = ld_relaxed(words + bd + static_cast<size_t>(k) * tstride);
        if (is_incl(vi)) break;
        if (vi != kEmpty) {
          ++k;
          continue;
        }
        if (++spins > kMaxSpin) {
          atomicAdd(ctrl + 1, 1u);
          lost = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (lost) {
        gend = __builtin_nanf("");
      } else {
        float gg = k < nTT ? hi_f(vi) : (dh_T ? dh_T[bd] : 0.0f);
        for (int jt = k - 1; jt > tt; --jt) {
          const unsigned long long va = ld_relaxed(words + bd + static_cast<size_t>(jt) * tstride);
          gg = is_incl(va) ? hi_f(va) : fmaf(lo_f(va), gg, hi_f(va));
        }
        gend = gg;
      }
      const float gstart = fmaf(At, gend, Ut);
      if (tt > 0)
        st_relaxed(words + bd + static_cast<size_t>(tt) * tstride, pack_incl(gstart));
      else if (dh0)
        dh0[bd] = gstart;
    }
    {
      float glo, ghi;
      halves(gend, glo, ghi);
      gend = glo;
    }
    // ---- pass 2: from g at this half's end, backward over its rows: gradients and sums
    float gk = half ? gend : fmaf(A1, gend, U1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next tile's staged rows landed
    float s_pa = 0.0f, s_px = 0.0f, s_rdz = 0.0f;
    // x~ of row jj is hi + lo of the conv tile (still intact: nothing writes it before the next
    // tile's conv)
    const bf16_t *xh = xa + (16 * half) * F::kLda + cl;
    const float hinit = h0 ? h0[static_cast<size_t>(b) * D + dc] : 0.0f;
    // dpre / dxc of sequence b as buffers: element (t0 + 16 half + jj, dc) at a wave-uniform row
    // offset (soffset) plus this lane's fixed offset. In the last tile of a sequence whose length
    // is not a multiple of the tile, rows at or past T get a lane offset past the buffer's end,
    // which the range check drops, and add nothing to the sums.
    const size_t sb = static_cast<size_t>(b) * T * D;
    const __amdgpu_buffer_rsrc_t rdp = __builtin_amdgcn_make_buffer_rsrc(
        wave_uniform(dpre + sb), static_cast<short>(0), rec_bytes(T, D, 4u), kRawWord3);
    const __amdgpu_buffer_rsrc_t rdx = __builtin_amdgcn_make_buffer_rsrc(
        wave_uniform(dxc + sb), static_cast<short>(0), rec_bytes(T, D, 2u), kRawWord3);
    const unsigned le = static_cast<unsigned>(16 * half * D + dc);
    auto pass2 = [&](auto nh, auto full) {
      // The LDS values of row jj (x~ hi and lo, dy, y) are loaded two rows ahead, and each row
      // is fenced off for the scheduler: left free it interleaves many rows and runs out of
      // registers.
      bf16_t hq[2], lq[2], dq[2], yq[2];
      auto fetch = [&](int jj) {
        hq[jj & 1] = xh[jj * F::kLda];
        lq[jj & 1] = xh[(kRows + jj) * F::kLda];
        dq[jj & 1] = dyt[jj * DH];
        yq[jj & 1] = yt[jj * DH];
      };
      fetch(15);
      fetch(14);
#pragma unroll
      for (int jj = 15; jj >= 0; --jj) {
        const int t = tl + jj;
        const bool in = decltype(full)::value || t < T;
        const float xc = bf16_to_f32(hq[jj & 1]) + bf16_to_f32(lq[jj & 1]);
        const float dyv = bf16_to_f32(dq[jj & 1]);
        const float yv = bf16_to_f32(yq[jj & 1]);
        if (jj >= 2) fetch(jj - 2);
        const float rr = acc[0][jj];
        const float ig = fast_sigmoid(acc[1][jj] + bx);
        const float e = ev[jj];
        const float a = 1.0f + e;
        const float m = __builtin_amdgcn_sqrtf(-e * (2.0f + e));
        const float delta = dyv + gk;
        const float hp = t > 0 ? yv : hinit;
        const float dx_ = delta * xc, dmg = delta * m;
        const float dm = dx_ * ig;
        const float di = dmg * xc;
        float dz = delta * hp * a;
        const float dr = dm * (a * a) * __builtin_amdgcn_rcpf(m);  // selected, not branched on
        dz -= m > 0.0f ? dr : 0.0f;
        const float dpa = kd * dz * (rr * (1.0f - rr));
        const float dpx = di * (ig * (1.0f - ig));
        s_pa += in ? dpa : 0.0f;
        s_px += in ? dpx : 0.0f;
        s_rdz = in ? fmaf(rr, dz, s_rdz) : s_rdz;
        gk = a * delta;
        const int so = static_cast<int>(row_bytes(t0 + jj, D, 1u));
        __builtin_amdgcn_raw_buffer_store_b32(pack_f16x2(dpa, dpx), rdp,
                                              static_cast<int>(in ? 4u * le : 0x80000000u), 4 * so, 0);
        __builtin_amdgcn_raw_buffer_store_b16(
            static_cast<uint16_t>(pack_f16x2(dmg * ig, 0.0f)), rdx,  // fp16
            static_cast<int>(in ? 2u * le : 0x80000000u), 2 * so, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (t0 + kRows <= T) {
      if (fast)
        pass2(std::true_type{}, std::true_type{});
      else
        pass2(std::false_type{}, std::true_type{});
    } else {
      if (fast)
        pass2(std::true_type{}, std::false_type{});
      else
        pass2(std::false_type{}, std::false_type{});
    }
    // ---- the tile's partial sums (half 0 + half 1), written by half 0
    {
      const size_t PD = static_cast<size_t>(B) * nTT * D;
      const size_t pidx = (static_cast<size_t>(b) * nTT + tt) * D + dc;
      float lo, hi;
      halves(s_pa, lo, hi);
      const float q0 = lo + hi;
      halves(s_px, lo, hi);
      const float q1 = lo + hi;
      halves(s_rdz, lo, hi);
      const float q2 = lo + hi;
      if (half == 0) {
        part[pidx] = q0;
        part[PD + pidx] = q1;
        part[2 * PD + pidx] = q2;
      }
    }
    cur ^= 1;
  }
}

// Look-back words to the empty pattern and the control words (give-up count, tickets) to 0
// before each launch.

// Look-back words to kEmpty, control words to 0.
__global__ void tile_bwd_reset(unsigned long long *slots, size_t n, unsigned *ctrl, int nctrl) {
  fill_lookback(slots, n, ctrl, nctrl);
}

bool fused_backward_supported(int Dh) { return Dh == 128 || Dh == 256; }

size_t fused_backward_slots(int B, int T, int D) {
  return static_cast<size_t>(B) * ((T + kRows - 1) / kRows) * D;  // one word per (tile, channel)
}

hipError_t launch_fused_backward(const void *x, const void *y, const void *dy, const float *h0,
                                 const float *dh_T, const void *conv_w, const void *W_a,
                                 const float *b_a, const void *W_x, const float *b_x,
                                 const float *Lambda, uint32_t *dpre, uint16_t *dxc,
                                 float *part, float *dh0, int B, int T, int D, int H,
                                 unsigned *ctrl, unsigned long long *slots, hipStream_t s) {
  const int nTT = (T + kRows - 1) / kRows;
  {
    const size_t n = fused_backward_slots(B, T, D);
    tile_bwd_reset<<<fill_blocks(n), 256, 0, s>>>(slots, n, ctrl, 2 + H);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // one workgroup per CU (the LDS of a tile), the same number for every head
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int per = std::max(1, std::min(cus / H, B * nTT));
  const bf16_t *xx = static_cast<const bf16_t *>(x);
  const bf16_t *yy = static_cast<const bf16_t *>(y);
  const bf16_t *dd = static_cast<const bf16_t *>(dy);
  const bf16_t *cw = static_cast<const bf16_t *>(conv_w);
  const bf16_t *wa = static_cast<const bf16_t *>(W_a);
  const bf16_t *wx = static_cast<const bf16_t *>(W_x);
  switch (D / H) {
    case 128:
      tile_bwd<128><<<H * per, BwdTile<128>::kThreads, 0, s>>>(
          xx, yy, dd, h0, dh_T, cw, wa, b_a, wx, b_x, Lambda, dpre, dxc, part, dh0, B, T, D,
          H, nTT, ctrl, slots);
      break;
    case 256:
      tile_bwd<256><<<H * per, BwdTile<256>::kThreads, 0, s>>>(
          xx, yy, dd, h0, dh_T, cw, wa, b_a, wx, b_x, Lambda, dpre, dxc, part, dh0, B, T, D,
          H, nTT, ctrl, slots);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rglru
