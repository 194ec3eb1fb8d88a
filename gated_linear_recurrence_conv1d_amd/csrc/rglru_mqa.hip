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
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators (P as bf16 hi + lo). The two waves of a pair
// split each block's keys for S and the softmax (32 keys each) and split dh for O (DH/2 columns
// each): per block they exchange the rows' maxima and then their P through LDS, so each wave
// holds half of O and does half of the softmax, fits in 256 registers, and two waves share each
// SIMD. The running max m and the rescales are the same in both waves of a pair (same inputs),
// each keeps the sum l over its own keys, and the two sums are added at the end. The k order
// inside a 16-key step follows the accumulator layout (keys 4h..4h+3 and 8+4h..8+4h+3 of half h);
// A and B use the same order, which is all a contraction needs. K and V are staged by direct
// buffer-to-LDS loads (K with its 16-byte chunks XOR-swizzled by row, V raw), double buffered:
// block j+1's loads are issued before block j's MFMAs. The V^T operand comes from row reads of
// DH/64 consecutive d per lane and key: O^T tile j of a wave holds the d columns
// (side) * DH/2 + (DH/64) * i + j, i = 0..31, and byte permutes pair two keys' values of one d.
#include "rglru_launch.h"
#include "rglru_mfma.h"

namespace rglru {

namespace {
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int kRawWord3 = 0x00020000;  // buffer descriptor word 3: raw 32-bit data, no swizzle
constexpr uint32_t kLoPair = 0x05040100u, kHiPair = 0x07060302u;  // low / high 16-bit halves
}  // namespace

template <int DH> struct Mqa {
  static_assert(DH == 64 || DH == 128 || DH == 256, "local MQA tile needs dh in {64, 128, 256}");
  static constexpr int kQB = 128;               // query rows per workgroup
  static constexpr int kKB = 64;                // keys per block
  static constexpr int kWaves = 8;              // 4 pairs x 32 rows; a wave = (pair, side)
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kKS = DH / 16;           // k-steps of S^T = K Q^T
  static constexpr int kDPL = DH / 64;          // d per lane per V row read = O^T tiles per wave
  static constexpr int kWPR = kDPL > 1 ? kDPL / 2 : 1;  // 32-bit words per V row read
  static constexpr int kDH2 = DH / 2;           // d columns of O per wave
  static constexpr int kCPR = DH / 8;           // 16-byte chunks per K row
  static constexpr int kRPI = 64 / kCPR;        // rows per wave-wide 16 B/lane load
  static constexpr int kKElems = kKB * DH;
  static constexpr int kBuf = 2 * kKElems;      // K then V, one block (bf16 elements)
  static constexpr int kLoads = kKB / kRPI;     // loads per block, each of K and V
  // P exchange: per wave 4 x 64 lanes x 16 B (hi and lo of its two 16-key steps). With DH = 256
  // it lives in the current block's K rows, which are dead once every wave has its S.
  static constexpr int kXpBytes = kWaves * 4 * 64 * 16;
  static constexpr bool kXpInK = kKElems * 2 >= kXpBytes;
  static constexpr int kXmBytes = kWaves * 32 * 4;  // per wave and row: max, at the end l
  static constexpr int kLdsBytes = 2 * kBuf * 2 + kXmBytes + (kXpInK ? 0 : kXpBytes);
};

template <int DH>
__global__ __launch_bounds__(Mqa<DH>::kThreads, 1) void local_mqa_fwd(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k, const bf16_t *__restrict__ v,
    bf16_t *__restrict__ o, int T, int Hq, int W, float c) {  // c = scale * log2(e)
  typedef Mqa<DH> M;
  __shared__ __attribute__((aligned(16))) unsigned char smem[M::kLdsBytes];
  bf16_t *lds = reinterpret_cast<bf16_t *>(smem);
  float *xm = reinterpret_cast<float *>(smem + 2 * M::kBuf * 2);
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int side = w & 1;           // keys 32 side.. of each block for S; d half for O
  const int lane = tid & 63;
  const int lrow = lane & 31;
  const int half = lane >> 5;
  const int q0 = blockIdx.x * M::kQB;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int qw = q0 + 32 * (w >> 1);  // the pair's first row
  const int qr = qw + lrow;           // this lane's row
  const size_t qstride = static_cast<size_t>(Hq) * DH;  // elements per position of q and o
  const bf16_t *kb_ = k + static_cast<size_t>(b) * T * DH;
  const bf16_t *vb_ = v + static_cast<size_t>(b) * T * DH;

  // the pair's Q rows: B operand of S^T = K Q^T (column = row qr, k = d)
  bf16x8_t qf[M::kKS];
  {
    const bf16_t *qp = q + (static_cast<size_t>(b) * T + min(qr, T - 1)) * qstride +
                       static_cast<size_t>(h) * DH + half * 8;
#pragma unroll
    for (int s = 0; s < M::kKS; ++s) qf[s] = load_bf16x8(qp + s * 16);
  }
  // keys this workgroup needs: [lo, hi]
  const int lo = max(0, q0 - W + 1);
  const int hi = min(T - 1, q0 + M::kQB - 1);
  const int kb_first = lo / M::kKB, kb_last = hi / M::kKB;

  // ---- staging, both by direct buffer-to-LDS loads (no registers; rows past T read zero: each
  // buffer covers exactly sequence b). K: rows of DH bf16 whose 16-byte chunks are XOR-swizzled
  // by the row's low 3 bits (chunk c of row r sits at c ^ (r & 7)), so that the A-operand reads of
  // 8 consecutive rows at one chunk hit 8 different chunk slots. V: raw rows.
  const __amdgpu_buffer_rsrc_t kseq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(kb_), static_cast<short>(0), T * DH * 2, kRawWord3);
  const __amdgpu_buffer_rsrc_t vseq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(vb_), static_cast<short>(0), T * DH * 2, kRawWord3);
  const int krow_l = lane / M::kCPR, kchunk_p = lane % M::kCPR;  // this lane's (row, slot)
  auto load_kv = [&](int kb, int buf) {
    bf16_t *Ks = lds + buf * M::kBuf;
    bf16_t *Vs = Ks + M::kKElems;
    for (int i = w; i < M::kLoads; i += M::kWaves) {
      const int row = i * M::kRPI + krow_l;
      const unsigned rowoff = static_cast<unsigned>((kb * M::kKB + row) * DH * 2);
      const unsigned koff = rowoff + static_cast<unsigned>((kchunk_p ^ (row & 7)) * 16);
      const unsigned voff = rowoff + static_cast<unsigned>(kchunk_p * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kseq, (lds_void_t *)(Ks + i * 512), 16, koff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vseq, (lds_void_t *)(Vs + i * 512), 16, voff, 0, 0, 0);
    }
  };

  f32x16_t oacc[M::kDPL];
#pragma unroll
  for (int j = 0; j < M::kDPL; ++j) oacc[j] = f32x16_t{};
  float m_run = -1e30f, l_run = 0.0f;  // finite start: fully masked blocks give p = 0, corr = 1

  load_kv(kb_first, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's rows landed
  __syncthreads();
  for (int kb = kb_first; kb <= kb_last; ++kb) {
    const int buf = (kb - kb_first) & 1;
    // the other buffer's readers finished before the barrier that ended kb - 1
    if (kb < kb_last) load_kv(kb + 1, buf ^ 1);
    const bf16_t *Ks = lds + buf * M::kBuf;
    const bf16_t *Vs = Ks + M::kKElems;
    u32x4_t *xp = reinterpret_cast<u32x4_t *>(
        M::kXpInK ? reinterpret_cast<unsigned char *>(lds + buf * M::kBuf)
                  : smem + 2 * M::kBuf * 2 + M::kXmBytes);
    const int K0 = kb * M::kKB, Ks0 = K0 + 32 * side;  // block start, this wave's first key
    // does any (key, row) pair of the pair's rows see each other in this block?
    const bool vis = K0 <= qw + 31 && K0 + M::kKB - 1 > qw - W && qw < T;
    f32x16_t sacc = f32x16_t{};
    float mx = -1e30f;
    if (vis) {
      // ---- S^T = K Q^T for this wave's 32 keys x 32 rows, one accumulator chain; the K
      // fragments are read two k-steps ahead of their MFMAs (pinned by the scheduling groups)
      auto kfrag = [&](int s) {
        const int r = 32 * side + lrow;
        return load_bf16x8(Ks + r * DH + (((2 * s + half) ^ (r & 7)) * 8));
      };
      bf16x8_t kf[3];
      kf[0] = kfrag(0);
      if (M::kKS > 1) kf[1] = kfrag(1);
#pragma unroll
      for (int s = 0; s < M::kKS; ++s) {
        if (s + 2 < M::kKS) kf[(s + 2) % 3] = kfrag(s + 2);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % 3], qf[s], sacc, 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, M::kKS > 1 ? 2 : 1, 0);  // steps 0, 1
#pragma unroll
      for (int s = 0; s < M::kKS; ++s) {
        if (s + 2 < M::kKS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // step s + 2
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      // step s
      }
      // ---- mask where some pair is out of the window, the causal order or the sequence
      const bool full = Ks0 + 31 <= qw && Ks0 > qw + 31 - W && Ks0 + 31 < T;
      if (!full) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = Ks0 + 8 * (j >> 2) + 4 * half + (j & 3);
          const bool ok = key <= qr && key > qr - W && key < T;
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
      mx = fmaxf(fmaxf(mq[0], mq[1]), mx);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (half == 0) xm[w * 32 + lrow] = mx;
    }
    __syncthreads();  // the partner's row maxima are in xm
    u32x4_t pown[4];  // this wave's P: (step 0 hi, lo, step 1 hi, lo)
    if (vis) {
      // ---- online softmax over the block's 64 keys (this wave's 32, the partner's row max).
      // O and l are kept relative to a running max m that is raised only when a block's max
      // exceeds it by more than 2^8 (in exp2 units) for some row of the wave: the rescale of the O
      // accumulators then happens about once per row instead of every block, and the
      // probabilities stay below 2^8. Numerator and denominator use the same m, so the result
      // does not change; both waves of the pair take the same decisions.
      mx = fmaxf(mx, xm[(w ^ 1) * 32 + lrow]);
      const bool raise = (mx - m_run) * c > 8.0f;
      if (__any(raise)) {  // wave-uniform
        const float m_new = raise ? mx : m_run;
        const float corr = __builtin_amdgcn_exp2f((m_run - m_new) * c);
        l_run *= corr;
        m_run = m_new;
#pragma unroll
        for (int j = 0; j < M::kDPL; ++j)
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
      // P as bf16 hi + lo (two MFMAs on the same V^T fragment): with P in bf16 alone, rows that
      // attend to few keys and whose output cancels (|o| well below its terms) lose ~1e-2 of the
      // output's rms
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = sacc[8 * st + 2 * e], p1 = sacc[8 * st + 2 * e + 1];
          const uint32_t hw = pack_bf16x2(p0, p1);
          pown[2 * st][e] = hw;
          pown[2 * st + 1][e] = pack_bf16x2(p0 - bf16lo(hw), p1 - bf16hi(hw));
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) xp[(w * 4 + i) * 64 + lane] = pown[i];
    }
    __syncthreads();  // the partner's P is in xp
    if (vis) {
      // ---- O^T += V^T P^T over the block's 4 steps of 16 keys; steps 2 side, 2 side + 1 are
      // this wave's own keys, the others the partner's (read back with the lane's own layout).
      // V^T operand of tile j: row i = d (side) * DH/2 + kDPL i + j, k = the step's 8 keys of
      // this half (kc..kc+3, kc+8..kc+11). Each lane reads kDPL consecutive d of each of the 8 key
      // rows (32 lanes cover the wave's DH/2 columns of one row) and pairs keys with byte permutes.
      const bf16_t *vcol = Vs + side * M::kDH2 + M::kDPL * lrow;
      auto vread = [&](int s4, uint32_t (&raw)[8][M::kWPR]) {
        const int kc = s4 * 16 + 4 * half;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const bf16_t *p = vcol + (kc + (r >> 2) * 8 + (r & 3)) * DH;
          if constexpr (M::kDPL == 4) {
            const uint2 t = *reinterpret_cast<const uint2 *>(p);
            raw[r][0] = t.x;
            raw[r][M::kWPR - 1] = t.y;
          } else if constexpr (M::kDPL == 2) {
            raw[r][0] = *reinterpret_cast<const uint32_t *>(p);
          } else {
            raw[r][0] = *reinterpret_cast<const unsigned short *>(p);
          }
        }
      };
      u32x4_t pother[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pother[i] = xp[((w ^ 1) * 4 + i) * 64 + lane];
      uint32_t raw[2][8][M::kWPR];  // one 16-key step ahead
      vread(0, raw[0]);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        if (s4 + 1 < 4) vread(s4 + 1, raw[(s4 + 1) & 1]);
        const bool own = (s4 >> 1) == side;
        const int st = s4 & 1;
        const bf16x8_t pfh = __builtin_bit_cast(bf16x8_t, own ? pown[2 * st] : pother[2 * st]);
        const bf16x8_t pfl = __builtin_bit_cast(bf16x8_t, own ? pown[2 * st + 1] : pother[2 * st + 1]);
#pragma unroll
        for (int j = 0; j < M::kDPL; ++j) {
          u32x4_t u;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            u[e] = __builtin_amdgcn_perm(raw[s4 & 1][2 * e + 1][j >> 1], raw[s4 & 1][2 * e][j >> 1],
                                         (j & 1) ? kHiPair : kLoPair);
          const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, u);
          oacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pfh, oacc[j], 0, 0, 0);
          oacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pfl, oacc[j], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next block's K and V rows landed
    __syncthreads();
  }
  // ---- l over the whole window: this wave's keys plus the partner's
  if (half == 0) xm[w * 32 + lrow] = l_run;
  __syncthreads();
  l_run += xm[(w ^ 1) * 32 + lrow];
  // ---- normalise and store. Lane = row qr; accumulator e of tile j is d = (half) * DH/2 +
  // kDPL r + j with r = 8 (e / 4) + 4 half + (e % 4), so for each g = e / 4 the lane holds
  // 4 kDPL consecutive d (position kDPL (e % 4) + j), stored as one run.
  if (qr < T) {
    const float inv = 1.0f / l_run;
    bf16_t *op = o + (static_cast<size_t>(b) * T + qr) * qstride + static_cast<size_t>(h) * DH +
                 side * M::kDH2;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t wv[2 * M::kDPL];
#pragma unroll
      for (int m = 0; m < 2 * M::kDPL; ++m) {
        const int p0 = 2 * m, p1 = 2 * m + 1;
        wv[m] = pack_bf16x2(oacc[p0 % M::kDPL][4 * g + p0 / M::kDPL] * inv,
                            oacc[p1 % M::kDPL][4 * g + p1 / M::kDPL] * inv);
      }
      bf16_t *dst = op + M::kDPL * (8 * g + 4 * half);
      if constexpr (M::kDPL == 1) {
        *reinterpret_cast<uint2 *>(dst) = make_uint2(wv[0], wv[1]);
      } else {
#pragma unroll
        for (int m = 0; m < 2 * M::kDPL; m += 4)
          *reinterpret_cast<uint4 *>(dst + 2 * m) = make_uint4(wv[m], wv[m + 1], wv[m + 2], wv[m + 3]);
      }
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
