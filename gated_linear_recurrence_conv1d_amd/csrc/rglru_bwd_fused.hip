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

// dpre / dlo / dxc / part / dh0 as the separate per-element kernel writes them (layouts in
// rglru_backward.hip); agg, incl: [nTT][B][D] words (each tile's map (A, U), and g at its start),
// all kEmpty; ctrl: [1] give-up count, [2 + g] head g's ticket, all 0.
template <int DH>
__global__ __launch_bounds__(BwdTile<DH>::kThreads, 1) void tile_bwd(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ y, const bf16_t *__restrict__ dy,
    const float *__restrict__ h0, const float *__restrict__ dh_T, const bf16_t *__restrict__ conv_w,
    const bf16_t *__restrict__ W_a, const float *__restrict__ b_a, const bf16_t *__restrict__ W_x,
    const float *__restrict__ b_x, const float *__restrict__ Lambda, uint32_t *__restrict__ dpre,
    uint32_t *__restrict__ dlo, float *__restrict__ dxc, float *__restrict__ part,
    float *__restrict__ dh0, int B, int T, int D, int H, int nTT, unsigned *ctrl,
    unsigned long long *agg, unsigned long long *incl) {
  typedef BwdTile<DH> F;
  __shared__ __attribute__((aligned(16))) bf16_t xr[2][F::kXRows * DH];  // x rows t0-3 ..
  __shared__ __attribute__((aligned(16))) bf16_t dyr[2][kRows * DH];     // dy rows t0 ..
  __shared__ __attribute__((aligned(16))) bf16_t yr[2][kRows * DH];      // y rows t0-1 ..
  __shared__ __attribute__((aligned(16))) bf16_t xa[2 * kRows * F::kLda];  // conv hi / lo; then pre
  __shared__ float2 sc[F::kSeg * DH];      // per (segment, channel): the segment's map (A, U)
  __shared__ float psum[3 * F::kSeg * DH];  // per (sum, segment, channel): partial sums
  __shared__ float gin[DH];                // g at the tile's end, per channel
  __shared__ int s_tile[2];
  uint32_t *const preL = reinterpret_cast<uint32_t *>(xa);  // [32][Dh] fp16 pairs (pa, px)

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lrow = lane & 31;
  const int half = lane >> 5;
  const int g = blockIdx.x % H;
  const int ntiles = B * nTT;
  unsigned *ticket = ctrl + 2 + g;
  // MFMA role: this lane's output channel, and its W_a / W_x rows (the B operand)
  const int cl = w * 32 + lrow;
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
  // conv role: channel pair cp (channels 2cp, 2cp + 1), tile rows cr * 16 .. + 15; lane-phase
  // role: channel c, rows sg * 32 .. + 31
  const int cp = tid % F::kPP;
  const int cr = tid / F::kPP;
  const int c = tid % DH;
  const int sg = tid / DH;
  const int dc = g * DH + c;
  // conv taps as bf16 pairs (w0, w1), (w2, w3): of the channel pair (conv role) and of channel c
  // (selector of its half of each pair: the lane phase reads the pair's staged words)
  bf16x2_t w01l, w23l, w01h, w23h, w01c, w23c;
  const uint32_t csel = (c & 1) ? kHiPair : kLoPair;
  {
    uint32_t cw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      cw[k] = *reinterpret_cast<const uint32_t *>(conv_w + static_cast<size_t>(k) * D + g * DH + 2 * cp);
    w01l = as_bf16x2(__builtin_amdgcn_perm(cw[1], cw[0], kLoPair));
    w23l = as_bf16x2(__builtin_amdgcn_perm(cw[3], cw[2], kLoPair));
    w01h = as_bf16x2(__builtin_amdgcn_perm(cw[1], cw[0], kHiPair));
    w23h = as_bf16x2(__builtin_amdgcn_perm(cw[3], cw[2], kHiPair));
#pragma unroll
    for (int k = 0; k < 4; ++k)
      cw[k] = *reinterpret_cast<const uint32_t *>(conv_w + static_cast<size_t>(k) * D + (dc & ~1));
    w01c = as_bf16x2(__builtin_amdgcn_perm(cw[1], cw[0], csel));
    w23c = as_bf16x2(__builtin_amdgcn_perm(cw[3], cw[2], csel));
  }
  const float kd = decay_coeff(Lambda[dc]);

  // conv of staged rows q .. q+3 (time t - 3 .. t for tile row q), as pair words: both channels
  // of the pair, or channel c alone
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
  auto conv1 = [&](const uint32_t (&xv)[4]) {
    return __builtin_amdgcn_fdot2_f32_bf16(
        as_bf16x2(__builtin_amdgcn_perm(xv[3], xv[2], csel)), w23c,
        __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(__builtin_amdgcn_perm(xv[1], xv[0], csel)), w01c,
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
        const_cast<bf16_t *>(x + so), static_cast<short>(0), T * D * 2, kRawWord3);
    const __amdgpu_buffer_rsrc_t sdy = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(dy + so), static_cast<short>(0), T * D * 2, kRawWord3);
    const __amdgpu_buffer_rsrc_t sy = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(y + so), static_cast<short>(0), T * D * 2, kRawWord3);
    for (int i = w; i < F::kLoads; i += F::kNW) {  // wave-uniform
      if (i < F::kXLoads) {
        const unsigned row_off = static_cast<unsigned>((t0 - 3 + i * F::kRowsPerLoad) * 2 * D);
        dma_16b(sx, row_off + lane_off, lds_addr(xr[bf] + i * F::kRowsPerLoad * DH));
      } else if (i < F::kXLoads + F::kRLoads) {
        const int q = i - F::kXLoads;
        const unsigned row_off = static_cast<unsigned>((t0 + q * F::kRowsPerLoad) * 2 * D);
        dma_16b(sdy, row_off + lane_off, lds_addr(dyr[bf] + q * F::kRowsPerLoad * DH));
      } else {
        const int q = i - F::kXLoads - F::kRLoads;
        const unsigned row_off = static_cast<unsigned>((t0 - 1 + q * F::kRowsPerLoad) * 2 * D);
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
  // explicitly (vmcnt(0) in pass 2, before the next tile's first barrier), and no global memory
  // is exchanged between the waves, so no barrier needs to wait for the y stores or the staging
  // loads in flight.
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
    // ---- [32 x DH] x [DH x 2 DH]: A = hi + lo
    f32x16_t acc[2];  // [gate]
    acc[0] = acc[1] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < F::kKS; ++ks)
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        const bf16x8_t af = load_bf16x8(xa + (pt * kRows + lrow) * F::kLda + ks * 16 + half * 8);
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, wa[ks], acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, wx[ks], acc[1], 0, 0, 0);
      }
    lds_barrier();  // every wave is done with xa
    // ---- pre-activations (with the biases) as fp16 pairs over the conv tile: row r, channel cl
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int r = 8 * (jj >> 2) + 4 * half + (jj & 3);
      preL[r * DH + cl] = pack_f16x2(acc[0][jj] + ba, acc[1][jj] + bx);
    }
    lds_barrier();  // pre ready
    // ---- lane phase, pass 1: this segment's map g_start = A g_end + U, walking it backward.
    // Rows at or past T (only in the last tile) are the identity (a = 1, dy = 0).
    const bf16_t *dyt = dyr[cur] + c;  // row r: dy at t0 + r
    const bf16_t *yt = yr[cur] + c;    // row r: y at t0 + r - 1 (zero for t0 + r - 1 < 0)
    const int rlast = sg * F::kSegRows + F::kSegRows - 1;  // the segment's last tile row
    float A = 1.0f, U = 0.0f;
#pragma unroll 4
    for (int row = rlast; row > rlast - F::kSegRows; --row) {
      const float pa = f16lo(preL[row * DH + c]);
      const bool in = t0 + row < T;
      const float a = in ? 1.0f + expm1_nonpos(kd * fast_sigmoid(pa)) : 1.0f;
      U = a * ((in ? bf16_to_f32(dyt[row * DH]) : 0.0f) + U);
      A *= a;
    }
    sc[sg * DH + c] = make_float2(A, U);
    lds_barrier();  // segment maps ready
    // ---- the tile's map, g at its end from the next tile in time, g at its start published
    if (sg == 0) {
      float At = 1.0f, Ut = 0.0f;
#pragma unroll
      for (int s = F::kSeg - 1; s >= 0; --s) {
        const float2 m = sc[s * DH + c];
        Ut = fmaf(m.x, Ut, m.y);
        At *= m.x;
      }
      // tile tt's words of this channel: agg (its map) and incl (g at its start), word k at
      // bd + k B D
      const size_t bd = static_cast<size_t>(b) * D + dc;
      const size_t tstride = static_cast<size_t>(B) * D;
      if (tt > 0) st_relaxed(agg + bd + static_cast<size_t>(tt) * tstride, pack2(At, Ut));
      // g at the tile's end is the fold g <- A_k g + U_k over the later tiles k, from dh_T at the
      // sequence end. Find the nearest later tile whose g_start is out, passing tiles whose map is
      // out (a map never waits for anything), then apply the maps in between in the fold's own
      // order: every incl word is an intermediate value of that one fold, so the result does not
      // depend on which words happened to be out (bitwise the same from run to run).
      float gend = 0.0f;
      int k = tt + 1;
      unsigned long long vi = kEmpty;
      unsigned spins = 0;
      bool lost = false;
      while (k < nTT) {
        vi = ld_relaxed(incl + bd + static_cast<size_t>(k) * tstride);
        if (vi != kEmpty) break;
        if (ld_relaxed(agg + bd + static_cast<size_t>(k) * tstride) != kEmpty) {
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
        float gg = k < nTT ? lo_f(vi) : (dh_T ? dh_T[bd] : 0.0f);
        for (int jt = k - 1; jt > tt; --jt) {
          const unsigned long long va = ld_relaxed(agg + bd + static_cast<size_t>(jt) * tstride);
          gg = fmaf(lo_f(va), gg, hi_f(va));
        }
        gend = gg;
      }
      const float gstart = fmaf(At, gend, Ut);
      if (tt > 0)
        st_relaxed(incl + bd + static_cast<size_t>(tt) * tstride, pack2(gstart, 0.0f));
      else if (dh0)
        dh0[bd] = gstart;
      gin[c] = gend;
    }
    lds_barrier();  // g at the tile's end ready
    // ---- pass 2: from g at this segment's end, backward over its rows: gradients and sums
    float gk = gin[c];
    for (int s = F::kSeg - 1; s > sg; --s) {
      const float2 m = sc[s * DH + c];
      gk = fmaf(m.x, gk, m.y);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next tile's staged rows landed
    float s_pa = 0.0f, s_px = 0.0f, s_rdz = 0.0f;
    // staged pair words of rows row .. row+3 (time t-3 .. t), slid down one row per step; start
    // with the rows above the segment's last row
    const bf16_t *xsc = xs + (c & ~1);
    uint32_t xv[4];
#pragma unroll
    for (int k = 0; k < 3; ++k) xv[k] = *reinterpret_cast<const uint32_t *>(xsc + (rlast + 1 + k) * DH);
    xv[3] = 0u;
    const size_t seq = static_cast<size_t>(b) * T * D;
    uint32_t *dpres = dpre + seq, *dlos = dlo + seq;
    float *dxcs = dxc + seq;
    const float hinit = h0 ? h0[static_cast<size_t>(b) * D + dc] : 0.0f;
#pragma unroll 4
    for (int row = rlast; row > rlast - F::kSegRows; --row) {
      const int t = t0 + row;
      xv[3] = xv[2];
      xv[2] = xv[1];
      xv[1] = xv[0];
      xv[0] = *reinterpret_cast<const uint32_t *>(xsc + row * DH);
      if (t < T) {
        const uint32_t pp = preL[row * DH + c];
        const float xc = conv1(xv);
        const float rr = fast_sigmoid(f16lo(pp));
        const float ig = fast_sigmoid(f16hi(pp));
        const float e = expm1_nonpos(kd * rr);
        const float a = 1.0f + e;
        const float m = __builtin_amdgcn_sqrtf(-e * (2.0f + e));
        const float delta = bf16_to_f32(dyt[row * DH]) + gk;
        const float hp = t > 0 ? bf16_to_f32(yt[row * DH]) : hinit;
        const float dx_ = delta * xc, dmg = delta * m;
        const float dm = dx_ * ig;
        const float di = dmg * xc;
        float dz = delta * hp * a;
        if (m > 0.0f) dz -= dm * (a * a) * __builtin_amdgcn_rcpf(m);
        const float dpa = kd * dz * (rr * (1.0f - rr));
        const float dpx = di * (ig * (1.0f - ig));
        s_pa += dpa;
        s_px += dpx;
        s_rdz = fmaf(rr, dz, s_rdz);
        gk = a * delta;
        const int o = t * D + dc;
        const uint32_t hpk = pack_bf16x2(dpa, dpx);
        dpres[o] = hpk;
        dlos[o] = pack_bf16x2(dpa - bf16lo(hpk), dpx - bf16hi(hpk));
        dxcs[o] = dmg * ig;
      }
    }
    psum[(0 * F::kSeg + sg) * DH + c] = s_pa;
    psum[(1 * F::kSeg + sg) * DH + c] = s_px;
    psum[(2 * F::kSeg + sg) * DH + c] = s_rdz;
    lds_barrier();  // partial sums ready
    if (sg == 0) {
      const size_t PD = static_cast<size_t>(B) * nTT * D;
      const size_t pidx = (static_cast<size_t>(b) * nTT + tt) * D + dc;
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        float sum = 0.0f;
#pragma unroll
        for (int s = 0; s < F::kSeg; ++s) sum += psum[(q * F::kSeg + s) * DH + c];
        part[q * PD + pidx] = sum;
      }
    }
    cur ^= 1;
  }
}

// Look-back words to the empty pattern and the control words (give-up count, tickets) to 0
// before each launch.
__global__ void tile_bwd_reset(unsigned long long *slots, size_t n, unsigned *ctrl, int nctrl) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    slots[i] = kEmpty;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nctrl; i += blockDim.x) ctrl[i] = 0u;
}

bool fused_backward_supported(int Dh) { return Dh == 128 || Dh == 256; }

size_t fused_backward_slots(int B, int T, int D) {
  return 2 * static_cast<size_t>(B) * ((T + kRows - 1) / kRows) * D;  // agg, then incl
}

hipError_t launch_fused_backward(const void *x, const void *y, const void *dy, const float *h0,
                                 const float *dh_T, const void *conv_w, const void *W_a,
                                 const float *b_a, const void *W_x, const float *b_x,
                                 const float *Lambda, uint32_t *dpre, uint32_t *dlo, float *dxc,
                                 float *part, float *dh0, int B, int T, int D, int H,
                                 unsigned *ctrl, unsigned long long *slots, hipStream_t s) {
  const int nTT = (T + kRows - 1) / kRows;
  unsigned long long *agg = slots, *incl = slots + fused_backward_slots(B, T, D) / 2;
  {
    const size_t n = fused_backward_slots(B, T, D);
    const unsigned blocks = static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 2048));
    tile_bwd_reset<<<std::max(1u, blocks), 256, 0, s>>>(slots, n, ctrl, 2 + H);
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
          xx, yy, dd, h0, dh_T, cw, wa, b_a, wx, b_x, Lambda, dpre, dlo, dxc, part, dh0, B, T, D,
          H, nTT, ctrl, agg, incl);
      break;
    case 256:
      tile_bwd<256><<<H * per, BwdTile<256>::kThreads, 0, s>>>(
          xx, yy, dd, h0, dh_T, cw, wa, b_a, wx, b_x, Lambda, dpre, dlo, dxc, part, dh0, B, T, D,
          H, nTT, ctrl, agg, incl);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rglru
