// rglru_mqa.hip -- local (sliding-window) multi-query attention, forward, bf16 on gfx950.
//
// Griffin's second temporal-mixing block (alby13 blog "Beyond Transformer Architecture: Griffin
// and Google RecurrentGemma", section "Core Components of Griffin -- 2. Local Sliding-Window
// MQA"): all query heads share one key/value head (multi-query), and each position attends only to
// a fixed window of recent positions, typically 1024, which bounds the KV cache; Soham De's Griffin
// thread (tweet on adding a local attention block every two recurrent blocks) has it capture the
// recent past while the RG-LRU carries the global state. Per sequence b, head h, position t:
//   o[b,t,h] = softmax_u(scale <q[b,t,h], k[b,u]>) v[b,u],  u in [max(0, t-W+1), t].
//
// One workgroup = 128 query rows of one (b, h), 8 waves in 4 pairs; a pair owns 32 rows and
// walks the 64-key blocks of the rows' windows. Both contractions put one query row in each lane:
//   S^T = K Q^T  (A = K rows from LDS, B = the pair's Q rows, in registers for the kernel's life),
//   O^T += V^T P^T (A = V^T from LDS, B = P),
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators (P as bf16 hi + lo where rows see few keys).
// The two waves of a pair split each block's keys for S and the softmax (32 keys each) and split
// dh for O (DH/2 columns each): per block they exchange the rows' maxima and then their P through
// LDS, so each wave
// holds half of O and does half of the softmax, fits in 256 registers, and two waves share each
// SIMD. The running max m and the rescales are the same in both waves of a pair (same inputs),
// each keeps the sum l over its own keys, and the two sums are added at the end.
//
// The lead pairs (waves 0-3) and the lagging pairs (waves 4-7) share the SIMDs one to one and run
// a third of a block apart, so that each SIMD has one wave's MFMAs beside the other's softmax.
// Per block, between three workgroup barriers:
//   segment A: lead S and row max          | lag softmax of the previous block
//   segment B: lead softmax                | lag P.V of the previous block
//   segment C: lead P.V                    | lag S and row max
// A wave's row maxima go into its partner's P-exchange slot, which the partner reads before it
// writes its own P there, so the exchange needs no space of its own.
//
// The k order inside a 16-key step follows the accumulator layout (keys 4h..4h+3 and
// 8+4h..8+4h+3 of half h); A and B use the same order, which is all a contraction needs. K and V
// are staged by direct buffer-to-LDS loads (16-byte chunks XOR-swizzled by row), two buffers each:
// block j's V rows arrive during segment A of block j, block j+1's K rows during segment B. The
// V^T operand comes from LDS by transposing reads (ds_read_b64_tr_b16: within each 16-lane group,
// lane i receives element i % 4 of the 8-byte pieces that lanes 4e + i / 4, e = 0..3, address),
// so that four lanes that read four consecutive key rows at 16 consecutive d hand each of 16 lanes
// one d over the four keys; the V rows' chunks are XOR-swizzled so that the 8 rows one read
// touches fall on different banks.
#include "rglru_launch.h"
#include "rglru_mfma.h"

#include <type_traits>

namespace rglru {

namespace {
constexpr int kRawWord3 = 0x00020000;  // buffer descriptor word 3: raw 32-bit data, no swizzle
constexpr unsigned kNoRows = 0x7F000000u;  // a byte offset past every sequence's K and V

}  // namespace

template <int DH> struct Mqa {
  static_assert(DH == 64 || DH == 128 || DH == 256, "local MQA tile needs dh in {64, 128, 256}");
  static constexpr int kQB = 128;               // query rows per workgroup
  static constexpr int kKB = 64;                // keys per block
  static constexpr int kWaves = 8;              // 4 pairs x 32 rows; a wave = (pair, side)
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kKS = DH / 16;           // k-steps of S^T = K Q^T
  static constexpr int kDT = DH / 64;           // 32-column O^T tiles per wave
  static constexpr int kDH2 = DH / 2;           // d columns of O per wave
  static constexpr int kCPR = DH / 8;           // 16-byte chunks per K row
  static constexpr int kRPI = 64 / kCPR;        // rows per wave-wide 16 B/lane load
  static constexpr int kKSw = kCPR < 16 ? kCPR - 1 : 15;  // K chunk swizzle mask
  static constexpr int kKElems = kKB * DH;      // one block of K (or V) rows, bf16 elements
  static constexpr int kLoads = kKB / kRPI;     // loads per block, each of K and V
  static constexpr int kLPW = kLoads / kWaves;  // ... per wave
  static_assert(kLoads % kWaves == 0 && kLPW <= kKS && kLPW <= 4, "loads spread over MFMAs");
  // LDS: K[2], V[2], then the P exchange: per wave 4 x 64 lanes x 16 B (hi and lo of its two
  // 16-key steps), whose first 128 bytes hold the partner's row maxima in between
  static constexpr int kXpBytes = kWaves * 4 * 64 * 16;
  static constexpr int kLdsBytes = 4 * kKElems * 2 + kXpBytes;
};

constexpr int kSplitKeys = 256;  // P as hi + lo below this many keys per row (see split)

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) float lds_float_t;

template <int DH>
__global__ __launch_bounds__(Mqa<DH>::kThreads, 1) void local_mqa_fwd(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k, const bf16_t *__restrict__ v,
    bf16_t *__restrict__ o, int T, int Hq, int W, float c) {  // c = scale * log2(e)
  typedef Mqa<DH> M;
  __shared__ __attribute__((aligned(16))) unsigned char smem[M::kLdsBytes];
  bf16_t *const Kbuf = reinterpret_cast<bf16_t *>(smem);  // [2][kKElems]
  bf16_t *const Vbuf = Kbuf + 2 * M::kKElems;              // [2][kKElems]
  // P exchange [8][4][64], as LDS pointers (a generic pointer would make these flat accesses,
  // which also wait for the outstanding vector memory loads)
  lds_u32x4_t *const xp = (lds_u32x4_t *)(smem + 4 * M::kKElems * 2);
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int side = w & 1;           // keys 32 side.. of each block for S; d half for O
  const bool lead = w < 4;
  const int lane = tid & 63;
  const int lrow = lane & 31;
  const int half = lane >> 5;
  // workgroups in order of decreasing work: query blocks from the last one down (a block near the
  // sequence start has fewer keys), all (sequence, head) pairs of one query block together, so that
  // the short ones fill the end of the launch
  const int nbh = gridDim.y * gridDim.z;
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int q0 = (gridDim.x - 1 - lin / nbh) * M::kQB;
  const int h = (lin % nbh) % Hq;
  const int b = (lin % nbh) / Hq;
  const int qw = q0 + 32 * (w >> 1);  // the pair's first row
  const int qr = qw + lrow;           // this lane's row
  const size_t qstride = static_cast<size_t>(Hq) * DH;  // elements per position of q and o
  const bf16_t *kb_ = k + static_cast<size_t>(b) * T * DH;
  const bf16_t *vb_ = v + static_cast<size_t>(b) * T * DH;
  // this wave's P-exchange slot (its P; before that, the partner's row maxima) and the partner's
  lds_u32x4_t *const xp_me = xp + w * 4 * 64;
  lds_u32x4_t *const xp_pa = xp + (w ^ 1) * 4 * 64;
  lds_float_t *const mx_in = (lds_float_t *)xp_me;   // the partner's maxima, for me
  lds_float_t *const mx_out = (lds_float_t *)xp_pa;  // my maxima, for the partner

  // the pair's Q rows: B operand of S^T = K Q^T (column = row qr, k = d)
  bf16x8_t qf[M::kKS];
  {
    const bf16_t *qp = q + (static_cast<size_t>(b) * T + min(qr, T - 1)) * qstride +
                       static_cast<size_t>(h) * DH + half * 8;
#pragma unroll
    for (int s = 0; s < M::kKS; ++s) qf[s] = load_bf16x8(qp + s * 16);
    // complete these loads here: inside the block loop the compiler does not see the LDS loads
    // (which share the vector memory counter) and would otherwise keep waiting on it for qf
#pragma unroll
    for (int s = 0; s < M::kKS; ++s) asm volatile("" ::"v"(qf[s]));
  }
  // P enters P.V as bf16 hi + lo only where some row of the workgroup sees fewer than
  // kSplitKeys keys (its first row: min(q0 + 1, W) keys). With more keys the rounding of P to
  // bf16 averages out below the output's rms (an fp64 emulation of B1 T2048 dh256 W1024: worst
  // element 8.4e-3 of the rms with bf16 P on rows with 256 keys or more, 3.9e-2 with bf16 P on
  // all rows, 3.9e-3 with hi + lo throughout), and the lo half's MFMAs -- a third of the
  // kernel's matrix work -- are skipped (a branch on a workgroup-uniform flag: a second copy of
  // the block loop without them spilled).
  const bool split = min(q0 + 1, W) < kSplitKeys;
  // keys this workgroup needs: [lo, hi]
  const int lo = max(0, q0 - W + 1);
  const int hi = min(T - 1, q0 + M::kQB - 1);
  const int kb_first = lo / M::kKB, kb_last = hi / M::kKB;

  // ---- staging by direct buffer-to-LDS loads (no registers; rows past T read zero: each buffer
  // covers exactly sequence b). K: chunk c of row r sits at c ^ (r & 15) (fewer bits when a row
  // has fewer chunks), so that the A-operand reads of 16 consecutive rows at one chunk, which the
  // LDS serves in one pass, hit 16 different chunk slots. V: chunk c of row r at c ^ 4 (r & 7)
  // (within the row), so that the 4-chunk runs of 8 consecutive rows fall on different banks.
  const __amdgpu_buffer_rsrc_t kseq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(kb_), static_cast<short>(0), T * DH * 2, kRawWord3);
  const __amdgpu_buffer_rsrc_t vseq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(vb_), static_cast<short>(0), T * DH * 2, kRawWord3);
  const int krow_l = lane / M::kCPR, kchunk_p = lane % M::kCPR;  // this lane's (row, slot)
  // this wave's ii-th load of block kb's K rows (or V rows) into buffer dst; kb < 0 fills dst
  // with zeros without touching memory (its offsets lie past the buffer's range). A wave that
  // issues many of these at once waits for the vector memory unit to take them, so they sit
  // between MFMAs or softmax work.
  auto load_rows = [&](bool isv, int ii, int kb, int dst_buf) {
    const int i = w + M::kWaves * ii;
    const int row = i * M::kRPI + krow_l;
    const unsigned rowoff = (kb < 0 ? kNoRows : static_cast<unsigned>(kb * M::kKB * DH * 2)) +
                            static_cast<unsigned>(row * DH * 2);
    const int sw = isv ? (4 * (row & 7)) & (M::kCPR - 1) : row & M::kKSw;
    const unsigned off = rowoff + static_cast<unsigned>((kchunk_p ^ sw) * 16);
    const bf16_t *dst = (isv ? Vbuf : Kbuf) + dst_buf * M::kKElems + i * 512;
    dma_16b(isv ? vseq : kseq, off,
            __builtin_amdgcn_readfirstlane(static_cast<unsigned>(reinterpret_cast<uintptr_t>(dst))));
  };

  f32x16_t oacc[M::kDT];
#pragma unroll
  for (int j = 0; j < M::kDT; ++j) oacc[j] = f32x16_t{};
  // transposing-read addresses (elements, relative to a block's V rows, step 0, first key
  // quad) of tile j: this lane reads key row 4 (lane / 32) + (lane % 16) / 4 at the d columns
  // (side) DH/2 + 32 j + 16 ((lane / 16) % 2) + 4 (lane % 4) .. + 3; it receives d =
  // (side) DH/2 + 32 j + lane % 32 over 4 consecutive keys
  // (chunk (d >> 3) ^ vsw = 4 ((side kDT + j) ^ (vsw / 4)) + (d >> 3) % 4, and side kDT + j =
  // side kDT | j: address = vbase + (vx ^ 32 j), one XOR-add per use)
  int vbase, vx;
  {
    const int vr = 4 * half + ((lane & 15) >> 2);  // row within the 8-row group (= row & 7)
    const int vsw = (4 * vr) & (M::kCPR - 1);
    const int d0 = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // d - (side) DH/2 - 32 j
    vbase = vr * DH + 8 * ((d0 >> 3) & 3) + (d0 & 7);
    vx = 32 * ((side * M::kDT) ^ (vsw >> 2));
  }
  float m_run = -1e30f, l_run = 0.0f;  // finite start: fully masked blocks give p = 0, corr = 1
  int kn = -1, kn_buf = 0;             // the K rows loading in segment B: block, buffer
  f32x16_t sacc = f32x16_t{};          // S^T of this wave's 32 keys, then their P
  float mx = -1e30f;                   // this block's row max over my keys
  u32x4_t pown[4];                     // my P: (step 0 hi, lo, step 1 hi, lo)

  // does any (key, row) pair of the pair's rows see each other in block kb?
  auto visible = [&](int kb) {
    const int K0 = kb * M::kKB;
    return K0 <= qw + 31 && K0 + M::kKB - 1 > qw - W && qw < T;
  };

  // ---- S^T = K Q^T for this wave's 32 keys x 32 rows of block kb, one accumulator chain (K
  // fragments read two k-steps ahead, pinned by scheduling groups, with the given loads between
  // the MFMAs), then the mask and the row max over my keys, stored for the partner
  auto block_s = [&](int kb, auto with_loads) {
    constexpr bool kLd = decltype(with_loads)::value;  // this block's V rows, between the MFMAs
    const bf16_t *Ks = Kbuf + (kb & 1) * M::kKElems;
    sacc = f32x16_t{};
    auto kfrag = [&](int s) {
      const int r = 32 * side + lrow;
      return load_bf16x8(Ks + r * DH + (((2 * s + half) ^ (r & M::kKSw)) * 8));
    };
    bf16x8_t kf[3];
    kf[0] = kfrag(0);
    if (M::kKS > 1) kf[1] = kfrag(1);
#pragma unroll
    for (int s = 0; s < M::kKS; ++s) {
      if (s + 2 < M::kKS) kf[(s + 2) % 3] = kfrag(s + 2);
      if (kLd && s < M::kLPW) load_rows(true, s, kb, kb & 1);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % 3], qf[s], sacc, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, M::kKS > 1 ? 2 : 1, 0);  // steps 0, 1
#pragma unroll
    for (int s = 0; s < M::kKS; ++s) {
      if (s + 2 < M::kKS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // step s + 2
      if (kLd && s < M::kLPW) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // a load
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      // step s
    }
    // mask where some pair is out of the window, the causal order or the sequence
    const int Ks0 = kb * M::kKB + 32 * side;
    const bool full = Ks0 + 31 <= qw && Ks0 > qw + 31 - W && Ks0 + 31 < T;
    if (!full) {
      // lane terms re-derived from the thread index here (this path is rare; kept live, they
      // would be spilled, and a reload waits for the loads in flight)
      const int tx = static_cast<int>(__builtin_amdgcn_workitem_id_x());
      const int rel = qw + (tx & 31) - Ks0 - 4 * ((tx >> 5) & 1);  // row - (key of j = 0)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int dk = 8 * (j >> 2) + (j & 3);  // key - (key of j = 0)
        const bool ok = dk <= rel && dk > rel - W && Ks0 + 4 * ((tx >> 5) & 1) + dk < T;
        sacc[j] = ok ? sacc[j] : -__builtin_inff();
      }
    }
    float mq[2];  // two independent chains
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      mq[i] = fmaxf(sacc[8 * i], sacc[8 * i + 1]);
#pragma unroll
      for (int j = 2; j < 8; ++j) mq[i] = fmaxf(mq[i], sacc[8 * i + j]);
    }
    mx = fmaxf(fmaxf(mq[0], mq[1]), -1e30f);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (half == 0) mx_out[lrow] = mx;
  };

  // ---- online softmax over the block's 64 keys (my 32, the partner's row max), then my P as
  // bf16 hi + lo into my exchange slot. O and l are kept relative to a running max m that is
  // raised only when a block's max exceeds it by more than 2^8 (in exp2 units) for some row of the
  // wave: the rescale of the O accumulators then happens about once per row instead of every
  // block, and the probabilities stay below 2^8. Numerator and denominator use the same m, so the
  // result does not change; both waves of the pair take the same decisions. With split, P enters
  // P.V as two MFMAs (hi, lo) on the same V^T fragment: with P in bf16 alone, rows that attend to
  // few keys and whose output cancels (|o| well below its terms) lose ~1e-2 of the output's rms.
  auto block_softmax = [&](auto with_loads, int kn) {
    constexpr bool kLd = decltype(with_loads)::value;  // block kn's K rows (kn < 0: zeros)
    const float m2 = fmaxf(mx, mx_in[lrow]);
    const bool raise = (m2 - m_run) * c > 8.0f;
    if (__any(raise)) {  // wave-uniform
      const float m_new = raise ? m2 : m_run;
      const float corr = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      l_run *= corr;
      m_run = m_new;
#pragma unroll
      for (int j = 0; j < M::kDT; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[j][e] *= corr;
    }
    const float mc = m_run * c;
    float pq[2] = {0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sacc[j], c, -mc));
      sacc[j] = p;
      pq[j >> 3] += p;
    }
    float ps = pq[0] + pq[1];
    ps += __shfl_xor(ps, 32, 64);
    l_run += ps;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = sacc[8 * st + 2 * e], p1 = sacc[8 * st + 2 * e + 1];
        const uint32_t hw = pack_bf16x2(p0, p1);
        pown[2 * st][e] = hw;
        pown[2 * st + 1][e] = pack_bf16x2(p0 - bf16lo(hw), p1 - bf16hi(hw));  // (unused unless split)
      }
    }
    if (kLd) {
#pragma unroll
      for (int ii = 0; ii < M::kLPW; ++ii) load_rows(false, ii, kn, kn_buf);
    }
    xp_me[lane] = pown[0];
    xp_me[2 * 64 + lane] = pown[2];
    if (split) {
      xp_me[64 + lane] = pown[1];
      xp_me[3 * 64 + lane] = pown[3];
    }
  };

  // ---- O^T += V^T P^T over block kb's 4 steps of 16 keys, my own two (steps 2 side, 2 side + 1)
  // first, then the partner's (read back with the lane's own layout). V^T operand of tile
  // j: row i = d (side) DH/2 + 32 j + i, k = the step's 8 keys of this half (kc..kc+3,
  // kc+8..kc+11), two transposing reads of 4 keys each. Loads of block kn's K rows sit between.
  auto block_pv = [&](int kb, auto with_loads, int kn) {
    constexpr bool kLd = decltype(with_loads)::value;
    const bf16_t *Vs = Vbuf + (kb & 1) * M::kKElems;
    auto vfrag = [&](int s4, int j) {
      const bf16_t *p = Vs + (vbase + (vx ^ (32 * j))) + s4 * 16 * DH;
      const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p);
      const i16x4_t c2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(p + 8 * DH));
      const uint2 ua = __builtin_bit_cast(uint2, a), uc = __builtin_bit_cast(uint2, c2);
      const u32x4_t u = {ua.x, ua.y, uc.x, uc.y};
      return __builtin_bit_cast(bf16x8_t, u);
    };
    bf16x8_t vf[2][M::kDT];  // read at the start of each step
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int st = t & 1;
      const int s4 = 2 * (t < 2 ? side : side ^ 1) + st;
#pragma unroll
      for (int j = 0; j < M::kDT; ++j) vf[t & 1][j] = vfrag(s4, j);
      if (kLd && t < M::kLPW) load_rows(false, t, kn, kn_buf);
      const bf16x8_t pfh =
          __builtin_bit_cast(bf16x8_t, t < 2 ? pown[2 * st] : xp_pa[(2 * st) * 64 + lane]);
#pragma unroll
      for (int j = 0; j < M::kDT; ++j)
        oacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t & 1][j], pfh, oacc[j], 0, 0, 0);
      if (split) {
        const bf16x8_t pfl = __builtin_bit_cast(
            bf16x8_t, t < 2 ? pown[2 * st + 1] : xp_pa[(2 * st + 1) * 64 + lane]);
#pragma unroll
        for (int j = 0; j < M::kDT; ++j)
          oacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t & 1][j], pfl, oacc[j], 0, 0, 0);
      }
    }
  };

  // ---- the block loop. Block kb's V rows go into V buffer kb & 1 during segment A (that
  // buffer's last reader, the lag's P.V of kb - 2, finished in segment B of kb - 1); block kb+1's
  // K rows into K buffer (kb+1) & 1 during segment B (its last reader, the lag's S of kb - 1,
  // finished in segment C of kb - 1). The exchange slots: maxima written in segment A (lead) or C
  // (lag) are read in the next segment, before the reader writes its P over them; P written in
  // segment B (lead) or A (lag) is read in the next segment.
#pragma unroll
  for (int ii = 0; ii < M::kLPW; ++ii) load_rows(false, ii, kb_first, kb_first & 1);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's K rows of the first block landed
  lds_barrier();
  bool pending = false;  // lag: the previous block's softmax and P.V are still to do
  const std::true_type loads;
  const std::false_type no_loads;
  for (int kb = kb_first; kb <= kb_last; ++kb) {
    const bool vis = visible(kb);
    kn = kb < kb_last ? kb + 1 : -1;  // block whose K rows load during segment B
    kn_buf = (kb + 1) & 1;
    // segment A
    if (lead) {
      if (vis) {
        block_s(kb, loads);
      } else {
#pragma unroll
        for (int ii = 0; ii < M::kLPW; ++ii) load_rows(true, ii, kb, kb & 1);
      }
    } else {
#pragma unroll
      for (int ii = 0; ii < M::kLPW; ++ii) load_rows(true, ii, kb, kb & 1);
      if (pending) block_softmax(no_loads, kn);
    }
    lds_barrier();
    // segment B
    if (lead) {
      if (vis) {
        block_softmax(loads, kn);
      } else {
#pragma unroll
        for (int ii = 0; ii < M::kLPW; ++ii) load_rows(false, ii, kn, kn_buf);
      }
    } else {
      if (pending) {
        block_pv(kb - 1, loads, kn);
      } else {
#pragma unroll
        for (int ii = 0; ii < M::kLPW; ++ii) load_rows(false, ii, kn, kn_buf);
      }
    }
    // this wave's V rows of block kb landed (its K loads of block kb+1, issued later, may not)
    __builtin_amdgcn_s_waitcnt(0x0F70 | (M::kLPW & 15));
    lds_barrier();
    // segment C
    if (lead) {
      if (vis) block_pv(kb, no_loads, kn);
    } else {
      if (vis) block_s(kb, no_loads);
      pending = vis;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's K rows of block kb+1 landed
    lds_barrier();
  }
  // the lag's last block
  if (!lead && pending) block_softmax(no_loads, kn);
  lds_barrier();
  if (!lead && pending) block_pv(kb_last, no_loads, kn);
  lds_barrier();
  // ---- l over the whole window: my keys plus the partner's
  if (half == 0) mx_out[lrow] = l_run;
  lds_barrier();
  l_run += mx_in[lrow];
  // ---- normalise and store. Lane = row qr; accumulator e of tile j is d = (side) DH/2 +
  // 32 j + 8 (e / 4) + 4 half + (e % 4): runs of 4 consecutive d.
  if (qr < T) {
    const float inv = 1.0f / l_run;
    bf16_t *op = o + (static_cast<size_t>(b) * T + qr) * qstride + static_cast<size_t>(h) * DH +
                 side * M::kDH2 + 4 * half;
#pragma unroll
    for (int j = 0; j < M::kDT; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint2 pk = make_uint2(pack_bf16x2(oacc[j][4 * g] * inv, oacc[j][4 * g + 1] * inv),
                                    pack_bf16x2(oacc[j][4 * g + 2] * inv, oacc[j][4 * g + 3] * inv));
        *reinterpret_cast<uint2 *>(op + 32 * j + 8 * g) = pk;
      }
  }
}

bool local_mqa_supported(int dh) { return dh == 64 || dh == 128 || dh == 256; }

hipError_t launch_local_mqa(const void *q, const void *k, const void *v, void *o, int B, int T,
                            int Hq, int dh, int window, float scale, hipStream_t s) {
  const float c = scale * 1.4426950408889634f;
  const dim3 grid((T + Mqa<64>::kQB - 1) / Mqa<64>::kQB, Hq, B);
  const bf16_t *qq = static_cast<const bf16_t *>(q);
  const bf16_t *kk = static_cast<const bf16_t *>(k);
  const bf16_t *vv = static_cast<const bf16_t *>(v);
  bf16_t *oo = static_cast<bf16_t *>(o);
  switch (dh) {
    case 64: local_mqa_fwd<64><<<grid, Mqa<64>::kThreads, 0, s>>>(qq, kk, vv, oo, T, Hq, window, c); break;
    case 128: local_mqa_fwd<128><<<grid, Mqa<128>::kThreads, 0, s>>>(qq, kk, vv, oo, T, Hq, window, c); break;
    case 256: local_mqa_fwd<256><<<grid, Mqa<256>::kThreads, 0, s>>>(qq, kk, vv, oo, T, Hq, window, c); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rglru
