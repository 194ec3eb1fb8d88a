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
//   1. conv in fp32 from x (3-row halo) into LDS (a bf16 copy as the MFMA A operand);
//   2. [64 x Dh] x [Dh x 2Dh] on v_mfma_f32_32x32x16_bf16, fp32 accumulators; the B operand is
//      this head's W_a / W_x rows, fetched per tile into registers (hot in L2);
//   3. gates elementwise in the accumulator layout -> (a, u) per element;
//   4. scan inside the tile: each lane owns one channel and four runs of 4 consecutive steps per
//      32-row tile, interleaved with its partner lane (lane ^ 32); in-lane scans of the runs,
//      then a chain over the 16 runs in time order with the partner's values fetched by lane swap;
//   5. decoupled look-back: publish the tile's aggregate (A, U) per channel, walk back over the
//      predecessor tiles of the same (sequence, head), combining aggregates until an inclusive
//      state (or the sequence start) is found, publish this tile's inclusive state;
//   6. fix-up h_t = P_t * carry + S_t and store y (and h_T for the last tile).
// Each published value is one 64-bit word (two fp32) written and read with relaxed agent-scope
// atomics, so no fences are needed; a small fill kernel resets the words to an all-ones
// "not yet" pattern (a NaN pair the kernel never writes) and the tickets to 0 before each launch.
// Because the look-back combines whatever predecessors have published so far, the association
// order of the carry (not the math) depends on timing: results are reproducible to the fp32
// rounding of the carried state, not bit for bit.
#include <algorithm>

#include "rglru_launch.h"
#include "rglru_mfma.h"

namespace rglru {

constexpr unsigned long long kEmpty = ~0ull;
constexpr int kFusedRows = 64;
constexpr unsigned kMaxSpin = 1u << 26;  // bounded wait: a lost predecessor yields NaN, not a hang

// A workgroup owns one head for its whole life (persistent) and walks that head's tiles in
// ticket order: one wave per 32 channels (8 waves for Dh = 256, two per SIMD, one workgroup per
// CU with a 100 KB LDS tile pair). Each wave keeps its channels' W_a / W_x rows -- the MFMA B
// operand, 128 VGPRs at Dh = 256 -- in registers for the whole kernel, so the tile loop touches
// HBM only for x and y. The conv of a tile is computed once, for all Dh channels.
template <int DH> struct Fused {
  static constexpr int kCPW = DH;                   // channels per workgroup
  static constexpr int kNW = kCPW / 32;             // waves
  static constexpr int kParts = DH / kCPW;          // workgroups per (sequence, head) tile
  static constexpr int kThreads = 64 * kNW;
  static constexpr int kKS = DH / 16;               // MFMA k-steps
  static constexpr int kLda = DH + 8;               // bf16 A-tile row stride (elements)
  static constexpr int kLdx = kCPW + 4;             // fp32 own-channel row stride (floats)
};

__device__ __forceinline__ unsigned long long pack2(float lo, float hi) {
  if (lo != lo) lo = __builtin_nanf("");
  return static_cast<unsigned long long>(__float_as_uint(lo)) |
         (static_cast<unsigned long long>(__float_as_uint(hi)) << 32);
}
__device__ __forceinline__ float lo_f(unsigned long long v) {
  return __uint_as_float(static_cast<uint32_t>(v));
}
__device__ __forceinline__ float hi_f(unsigned long long v) {
  return __uint_as_float(static_cast<uint32_t>(v >> 32));
}
__device__ __forceinline__ unsigned long long ld_relaxed(const unsigned long long *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(unsigned long long *p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

// Control words: [0] unused, [1] count of lanes that gave up waiting (diagnostic), [2 + p] the
// tile ticket of (head, part) pair p.
__global__ void fused_reset(unsigned long long *slots, size_t n, unsigned *ctrl, int nctrl) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    slots[i] = kEmpty;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nctrl; i += blockDim.x) ctrl[i] = 0u;
}

struct TileCtx {
  int j, tt, b, t0;
};

// Gates, in-tile scan, look-back and output for one tile (accumulators in, y out). Rows past the
// end of the sequence (only in the last tile) are computed like the others from zero input --
// they come after every real row, so they cannot change a real row's state -- and only their
// stores are masked; h_T is then taken at row T-1 instead of at the end of the tile.
template <int DH>
__device__ __forceinline__ void fused_epilogue(
    f32x16_t (&acc)[2][2], const float *xf, int xcol, int lane, const TileCtx &tc, int g, int cl,
    int d, float kd, float ba2, float bx2, const float *__restrict__ h0, bf16_t *__restrict__ y,
    float *__restrict__ h_T, int B, int T, int D, int H, int nTT, unsigned *ctrl,
    unsigned long long *agg, unsigned long long *incl) {
  typedef Fused<DH> F;
  const int half = lane >> 5;
  const int lrow = lane & 31;
  // Accumulator jj of this lane holds tile row rt*32 + 8*(jj/4) + 4*half + (jj%4): run
  // k = rt*4 + jj/4 covers 4 consecutive rows; in time order the runs alternate between the
  // halves (run index 2k + half).
  // (a) recurrence gate -> z = log a, overwriting the pa accumulator; track the smallest z.
  float zmin = 0.0f;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const float r = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(acc[rt][0][jj] + ba2));
      const float z = kd * r;
      acc[rt][0][jj] = z;
      zmin = fminf(zmin, z);
      if ((jj & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
  // expm1 leaves its Taylor range only for fast decays; test once per tile for the whole wave.
  const bool wide = __any(zmin < -0.25f);
  // (b) input gate, normaliser, runs of 4 steps, and the chain over the 16 runs in time order:
  // this lane's run k pairs with the partner half's run k (runs 2k and 2k+1 of the tile).
  float cz[8], qz[8];  // per own run: state from 0 at its start, product of a before it
  float c = 0.0f, qp = 1.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int rt = k >> 2, jb = k & 3;
    float Pp = 1.0f, S = 0.0f;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int jj = jb * 4 + e4;
      const int row = rt * 32 + 8 * jb + 4 * half + e4;
      const float z = acc[rt][0][jj];
      float e = expm1_poly(z);
      if (wide) {
        if (z < -0.25f) e = __builtin_amdgcn_exp2f(z * kLog2e) - 1.0f;
      }
      const float a = 1.0f + e;
      const float m = __builtin_amdgcn_sqrtf(-e * (2.0f + e));
      const float ig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(acc[rt][1][jj] + bx2));
      const float u = m * (ig * xf[row * F::kLdx + xcol]);
      S = fmaf(a, S, u);
      Pp *= a;
      acc[rt][0][jj] = Pp;  // prefix product within the run
      acc[rt][1][jj] = S;   // state within the run from 0
    }
    const float pa_ = __shfl_xor(Pp, 32, 64);
    const float pu_ = __shfl_xor(S, 32, 64);
    const float A0 = half ? pa_ : Pp, U0 = half ? pu_ : S;
    const float A1 = half ? Pp : pa_, U1 = half ? S : pu_;
    const float c1 = fmaf(A0, c, U0), q1 = qp * A0;  // start of run 2k+1
    cz[k] = half ? c1 : c;
    qz[k] = half ? q1 : qp;
    c = fmaf(A1, c1, U1);
    qp = q1 * A1;
    // keep the scheduler from hoisting later runs' loads and transcendentals (live ranges)
    __builtin_amdgcn_sched_barrier(0);
  }
  const float At = qp, Ut = c;  // the tile as one affine map of this channel

  // (d) decoupled look-back on half 0 (one channel per lane).
  float h_in = 0.0f;
  if (half == 0) {
    const size_t slot = (static_cast<size_t>(tc.j) * H + g) * DH + cl;  // j = tt*B + b
    if (tc.tt + 1 < nTT) st_relaxed(agg + slot, pack2(At, Ut));
    const float hstart = h0 ? h0[static_cast<size_t>(tc.b) * D + d] : 0.0f;
    if (tc.tt == 0) {
      h_in = hstart;
    } else {
      float Aacc = 1.0f, Uacc = 0.0f;
      int jt = tc.tt - 1;
      unsigned spins = 0;
      for (;;) {
        const size_t ps = ((static_cast<size_t>(jt) * B + tc.b) * H + g) * DH + cl;
        const unsigned long long vi = ld_relaxed(incl + ps);
        if (vi != kEmpty) {
          h_in = fmaf(Aacc, lo_f(vi), Uacc);
          break;
        }
        const unsigned long long va = ld_relaxed(agg + ps);
        if (va != kEmpty) {
          Uacc = fmaf(Aacc, hi_f(va), Uacc);
          Aacc *= lo_f(va);
          if (--jt < 0) {
            h_in = fmaf(Aacc, hstart, Uacc);
            break;
          }
          continue;
        }
        if (++spins > kMaxSpin) {
          atomicAdd(ctrl + 1, 1u);
          h_in = __builtin_nanf("");
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    const float h_end = fmaf(At, h_in, Ut);
    if (tc.tt + 1 < nTT)
      st_relaxed(incl + slot, pack2(h_end, 0.0f));
    else if (h_T && tc.t0 + kFusedRows == T)
      h_T[static_cast<size_t>(tc.b) * D + d] = h_end;
  }
  h_in = __shfl(h_in, lrow, 64);

  // (e) fix-up and store y. Row addresses are wave-uniform: a scalar row pointer plus the lane's
  // 32-bit offset (its channel and its half's 4-row shift). Dv is re-materialised through an
  // empty asm so that the compiler cannot hoist the 32 row offsets out of the tile loop (it
  // would keep them in VGPRs, spill them and reload one per store).
  unsigned Dv = static_cast<unsigned>(D);
  asm volatile("" : "+s"(Dv));
  bf16_t *yt = y + (static_cast<size_t>(tc.b) * T + tc.t0) * D;  // this tile's row 0
  const unsigned lane_off = static_cast<unsigned>(d - g * DH) + 4u * half * Dv;
  char *yh = reinterpret_cast<char *>(yt + g * DH);
  float carry[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) carry[k] = fmaf(qz[k], h_in, cz[k]);
  if (tc.t0 + kFusedRows <= T) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int r = rt * 32 + 8 * (jj >> 2) + (jj & 3);  // row of half 0; half 1: 4 further
        const float hv = fmaf(acc[rt][0][jj], carry[rt * 4 + (jj >> 2)], acc[rt][1][jj]);
        *reinterpret_cast<bf16_t *>(yh + (r * Dv + lane_off) * 2u) = f32_to_bf16(hv);
      }
  } else {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int r = rt * 32 + 8 * (jj >> 2) + (jj & 3);
        const float hv = fmaf(acc[rt][0][jj], carry[rt * 4 + (jj >> 2)], acc[rt][1][jj]);
        const int t = tc.t0 + r + 4 * half;
        if (t < T) *reinterpret_cast<bf16_t *>(yh + (r * Dv + lane_off) * 2u) = f32_to_bf16(hv);
        if (t == T - 1 && h_T) h_T[static_cast<size_t>(tc.b) * D + d] = hv;
      }
  }
}

template <int DH>
__global__ __launch_bounds__(Fused<DH>::kThreads, 2) void fused_forward(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ conv_w,
    const bf16_t *__restrict__ W_a, const float *__restrict__ b_a,
    const bf16_t *__restrict__ W_x, const float *__restrict__ b_x,
    const float *__restrict__ Lambda, const float *__restrict__ h0, bf16_t *__restrict__ y,
    float *__restrict__ h_T, int B, int T, int D, int H, int nTT, unsigned *ctrl,
    unsigned long long *agg, unsigned long long *incl) {
  typedef Fused<DH> F;
  // A tile: bf16(-log2(e) * conv output), so the accumulators come out in log2 units and the
  // sigmoids need no extra multiply (the bf16 rounding error is the same as for the plain conv
  // output). xf: the plain fp32 conv output of this part's channels, for the input term.
  __shared__ __attribute__((aligned(16))) bf16_t xa[kFusedRows * F::kLda];
  __shared__ __attribute__((aligned(16))) float xf[kFusedRows * F::kLdx];
  __shared__ int s_tile[2];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int lrow = lane & 31;
  const int half = lane >> 5;
  const int P2 = H * F::kParts;
  const int pair = blockIdx.x % P2;
  const int g = pair / F::kParts;
  const int part = pair % F::kParts;
  const int ntiles = B * nTT;
  unsigned *ticket = ctrl + 2 + pair;
  const int xcol = w * 32 + lrow;           // this lane's channel within the part
  const int cl = part * F::kCPW + xcol;     // ... within the head
  const int d = g * DH + cl;
  const float kd = decay_coeff(Lambda[d]);
  const float ba2 = -kLog2e * b_a[d], bx2 = -kLog2e * b_x[d];
  // B operand of this wave: its 32 channels' W_a / W_x rows, resident for the kernel's life
  bf16x8_t wa[F::kKS], wx[F::kKS];
  {
    const bf16_t *wa_row = W_a + (static_cast<size_t>(g) * DH + cl) * DH + half * 8;
    const bf16_t *wx_row = W_x + (static_cast<size_t>(g) * DH + cl) * DH + half * 8;
#pragma unroll
    for (int ks = 0; ks < F::kKS; ++ks) {
      wa[ks] = load_bf16x8(wa_row + ks * 16);
      wx[ks] = load_bf16x8(wx_row + ks * 16);
    }
  }

  // conv-prologue role of this thread: channel pair pc0/pc0+1, rows pr0 .. pr0+PRPG-1
  constexpr int PP = DH / 2;
  constexpr int PRPG = kFusedRows * PP / F::kThreads;
  constexpr int PSUB = PRPG > 16 ? 16 : PRPG;  // rows per load batch (bounds live registers)
  const int pc0 = 2 * (tid % PP);
  // a wave spans whole row groups only when a row group is >= 64 lanes wide (Dh >= 128); then
  // the row index is wave-uniform and all row arithmetic stays scalar
  const int pr0 = PP % 64 == 0 ? __builtin_amdgcn_readfirstlane((tid / PP) * PRPG)
                               : (tid / PP) * PRPG;
  const int pd0 = g * DH + pc0;
  const int pcf = pc0 - part * F::kCPW;
  const bool pmine = __builtin_amdgcn_readfirstlane(pcf >= 0 && pcf < F::kCPW);  // per wave

  for (int it = 0;; ++it) {
    if (tid == 0) s_tile[it & 1] = static_cast<int>(atomicAdd(ticket, 1u));
    __syncthreads();
    TileCtx tc;
    tc.j = __builtin_amdgcn_readfirstlane(s_tile[it & 1]);
    if (tc.j >= ntiles) break;
    tc.tt = tc.j / B;
    tc.b = tc.j % B;
    tc.t0 = tc.tt * kFusedRows;

    // ---- conv prologue (fp32). Thread = (channel pair p, run of rows r0..). Every load is
    // unconditional so that all of them are in flight at once: row indices past the end are
    // clamped to T-1 (those rows only feed rows >= T, whose results are discarded), and the three
    // halo rows before t = 0 are zeroed by a wave-uniform branch in the first tile only.
    // Offsets within one sequence fit in 32 bits (T * D < 2^31 is checked by the launcher).
    {
      uint32_t cw[4];  // the pair's conv taps (bf16x2); re-read per tile (cache hits) to save VGPRs
#pragma unroll
      for (int k = 0; k < 4; ++k)
        cw[k] = *reinterpret_cast<const uint32_t *>(conv_w + static_cast<size_t>(k) * D + pd0);
      const char *xb = reinterpret_cast<const char *>(x + static_cast<size_t>(tc.b) * T * D);
#pragma unroll
      for (int rb = 0; rb < PRPG; rb += PSUB) {
        uint32_t xv[PSUB + 3];
#pragma unroll
        for (int k = 0; k < PSUB + 3; ++k) {
          const int t = min(max(tc.t0 + pr0 + rb - 3 + k, 0), T - 1);  // scalar
          xv[k] = *reinterpret_cast<const uint32_t *>(xb + static_cast<unsigned>(t * D) * 2u +
                                                      static_cast<unsigned>(pd0) * 2u);
        }
        if (tc.t0 + pr0 + rb == 0) {  // wave-uniform
          xv[0] = 0u;
          xv[1] = 0u;
          xv[2] = 0u;
        }
#pragma unroll
        for (int r = 0; r < PSUB; ++r) {
          const float o0 = fmaf(bf16lo(cw[3]), bf16lo(xv[r + 3]),
                                fmaf(bf16lo(cw[2]), bf16lo(xv[r + 2]),
                                     fmaf(bf16lo(cw[1]), bf16lo(xv[r + 1]),
                                          bf16lo(cw[0]) * bf16lo(xv[r]))));
          const float o1 = fmaf(bf16hi(cw[3]), bf16hi(xv[r + 3]),
                                fmaf(bf16hi(cw[2]), bf16hi(xv[r + 2]),
                                     fmaf(bf16hi(cw[1]), bf16hi(xv[r + 1]),
                                          bf16hi(cw[0]) * bf16hi(xv[r]))));
          const int row = pr0 + rb + r;
          *reinterpret_cast<uint32_t *>(xa + row * F::kLda + pc0) =
              pack_bf16x2(-kLog2e * o0, -kLog2e * o1);
          if (pmine) *reinterpret_cast<float2 *>(xf + row * F::kLdx + pcf) = make_float2(o0, o1);
        }
      }
    }
    __syncthreads();

    // ---- gate projections on MFMA: 64 rows x (32 channels x 2 gates) per wave.
    f32x16_t acc[2][2];  // [row tile][gate]
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      acc[rt][0] = f32x16_t{};
      acc[rt][1] = f32x16_t{};
    }
#pragma unroll
    for (int ks = 0; ks < F::kKS; ++ks) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const bf16x8_t af = load_bf16x8(xa + (rt * 32 + lrow) * F::kLda + ks * 16 + half * 8);
        acc[rt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, wa[ks], acc[rt][0], 0, 0, 0);
        acc[rt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, wx[ks], acc[rt][1], 0, 0, 0);
      }
    }

    fused_epilogue<DH>(acc, xf, xcol, lane, tc, g, cl, d, kd, ba2, bx2, h0, y, h_T, B, T, D, H,
                       nTT, ctrl, agg, incl);
  }
}

size_t fused_ctrl_bytes(int H) { return (static_cast<size_t>(2 + 2 * H) * 4 + 255) / 256 * 256; }

size_t fused_slots(int B, int T, int H, int Dh) {
  const size_t nTT = (T + kFusedRows - 1) / kFusedRows;
  return nTT * B * H * Dh;
}

bool fused_supported(int io, int T, int D, int Dh) {
  return io == kBF16 && (Dh == 32 || Dh == 64 || Dh == 128 || Dh == 256) &&
         static_cast<long long>(T) * D < (1LL << 31);
}

hipError_t launch_fused(const void *x, const void *conv_w, const void *W_a, const float *b_a,
                        const void *W_x, const float *b_x, const float *Lambda, const float *h0,
                        void *y, float *h_T, int B, int T, int D, int H, void *ctrl_ws,
                        hipStream_t s) {
  const int Dh = D / H;
  const int nTT = (T + kFusedRows - 1) / kFusedRows;
  const size_t nslot = fused_slots(B, T, H, Dh);
  unsigned *ctrl = static_cast<unsigned *>(ctrl_ws);
  unsigned long long *agg =
      reinterpret_cast<unsigned long long *>(static_cast<char *>(ctrl_ws) + fused_ctrl_bytes(H));
  unsigned long long *incl = agg + nslot;
  const unsigned rblocks = static_cast<unsigned>(std::min<size_t>((2 * nslot + 255) / 256, 4096));
  fused_reset<<<rblocks, 256, 0, s>>>(agg, 2 * nslot, ctrl, 2 + 2 * H);
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
    const int P2 = H * Fused<DHV>::kParts;                                                      \
    const int per = std::max(1, (cus + P2 - 1) / P2);                                       \
    fused_forward<DHV><<<P2 * per, Fused<DHV>::kThreads, 0, s>>>(                               \
        xx, cw, wa, b_a, wx, b_x, Lambda, h0, yy, h_T, B, T, D, H, nTT, ctrl, agg, incl);       \
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

}  // namespace rglru
