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
// One workgroup = 128 query rows of one (b, h), 4 waves of 32 rows; it walks the 64-key blocks
// of the rows' windows. Both contractions are laid out so that a lane owns one query row:
//   S^T = K Q^T  (A = K rows from LDS, B = the wave's Q rows, in registers for the kernel's life),
//   O^T += V^T P^T (A = V^T rows from LDS, B = P taken straight from the S^T accumulators),
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators (P as bf16 hi + lo). The online softmax (running max m, sum l, the
// rescale of O) is then lane-local apart from one exchange with the partner half-wave, which holds
// the other half of the row's keys. The k order inside a 16-key step follows the accumulator
// layout (keys 4h..4h+3 and 8+4h..8+4h+3 of half h); A and B use the same order, which is all a
// contraction needs. K and V are staged by direct buffer-to-LDS loads (K with its 16-byte chunks
// XOR-swizzled by row, V raw, read as 2-byte pieces for the V^T operand), double buffered: block
// j+1's loads are issued before block j's MFMAs.
#include "rglru_launch.h"
#include "rglru_mfma.h"

namespace rglru {

namespace {
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int kRawWord3 = 0x00020000;  // buffer descriptor word 3: raw 32-bit data, no swizzle
}  // namespace

template <int DH> struct Mqa {
  static_assert(DH == 64 || DH == 128 || DH == 256, "local MQA tile needs dh in {64, 128, 256}");
  static constexpr int kQB = 128;               // query rows per workgroup
  static constexpr int kKB = 64;                // keys per block
  static constexpr int kThreads = 256;          // 4 waves x 32 rows
  static constexpr int kKS = DH / 16;           // k-steps of S^T = K Q^T
  static constexpr int kDT = DH / 32;           // 32-row d tiles of O^T
  static constexpr int kLdK = DH;               // bf16 per K row (16-byte chunks XOR-swizzled)
  static constexpr int kCPR = DH / 8;           // 16-byte chunks per K row
  static constexpr int kRPI = 64 / kCPR;        // K rows per wave-wide 16 B/lane load
  static constexpr int kLdV = DH;               // bf16 per V row (raw, as in HBM)
  static constexpr int kKElems = kKB * kLdK;
  static constexpr int kVElems = kKB * kLdV;
  static constexpr int kBuf = kKElems + kVElems;
  static constexpr int kKLoads = kKB / kRPI;                    // K loads per block
};

__device__ __forceinline__ bf16x8_t lds_read_4x2(const bf16_t *p0, const bf16_t *p1) {
  const uint2 a = *reinterpret_cast<const uint2 *>(p0);
  const uint2 b = *reinterpret_cast<const uint2 *>(p1);
  const u32x4_t v = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(bf16x8_t, v);
}

template <int DH>
__global__ __launch_bounds__(Mqa<DH>::kThreads, 1) void local_mqa_fwd(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k, const bf16_t *__restrict__ v,
    bf16_t *__restrict__ o, int T, int Hq, int W, float c) {  // c = scale * log2(e)
  typedef Mqa<DH> M;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * M::kBuf];
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int lrow = lane & 31;
  const int half = lane >> 5;
  const int q0 = blockIdx.x * M::kQB;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int qw = q0 + 32 * w;       // this wave's first row
  const int qr = qw + lrow;         // this lane's row
  const size_t qstride = static_cast<size_t>(Hq) * DH;  // elements per position of q and o
  const bf16_t *kb_ = k + static_cast<size_t>(b) * T * DH;
  const bf16_t *vb_ = v + static_cast<size_t>(b) * T * DH;

  // the wave's Q rows: B operand of S^T = K Q^T (column = row qr, k = d)
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
  // 8 consecutive rows at one chunk hit 8 different chunk slots. V: raw rows; the O^T contraction
  // reads its A operand (V^T: one d, 8 keys) as 2-byte reads, 32 lanes on consecutive d.
  const __amdgpu_buffer_rsrc_t kseq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(kb_), static_cast<short>(0), T * DH * 2, kRawWord3);
  const __amdgpu_buffer_rsrc_t vseq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(vb_), static_cast<short>(0), T * DH * 2, kRawWord3);
  const int krow_l = lane / M::kCPR, kchunk_p = lane % M::kCPR;  // this lane's (row, slot)
  auto load_kv = [&](int kb, int buf) {
    bf16_t *Ks = lds + buf * M::kBuf;
    bf16_t *Vs = Ks + M::kKElems;
    for (int i = w; i < M::kKLoads; i += 4) {
      const int row = i * M::kRPI + krow_l;
      const unsigned rowoff = static_cast<unsigned>((kb * M::kKB + row) * DH * 2);
      const unsigned koff = rowoff + static_cast<unsigned>((kchunk_p ^ (row & 7)) * 16);
      const unsigned voff = rowoff + static_cast<unsigned>(kchunk_p * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kseq, (lds_void_t *)(Ks + i * 512), 16, koff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vseq, (lds_void_t *)(Vs + i * 512), 16, voff, 0, 0, 0);
    }
  };

  f32x16_t oacc[M::kDT];
#pragma unroll
  for (int dt = 0; dt < M::kDT; ++dt) oacc[dt] = f32x16_t{};
  float m_run = -1e30f, l_run = 0.0f;  // finite start: fully masked blocks give p = 0, corr = 1

  load_kv(kb_first, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's rows landed
  __syncthreads();
  for (int kb = kb_first; kb <= kb_last; ++kb) {
    const int buf = (kb - kb_first) & 1;
    const bool more = kb < kb_last;
    // the other buffer's readers finished before the barrier that ended kb - 1
    if (more) load_kv(kb + 1, buf ^ 1);
    const int K0 = kb * M::kKB, K1 = K0 + M::kKB - 1;
    const int Q0 = qw, Q1 = qw + 31;
    // does any (key, row) pair of this wave see each other in this block?
    if (K0 <= Q1 && K1 > Q0 - W && Q0 < T) {
      const bf16_t *Ks = lds + buf * M::kBuf;
      const bf16_t *Vs = Ks + M::kKElems;
      // ---- S^T = K Q^T: 64 keys x 32 rows; K fragments read two k-steps ahead of their MFMAs
      // (one wave per SIMD: nothing else would hide the LDS latency)
      // four accumulator chains (row tile x k-step parity): an MFMA never waits on the one
      // before it
      f32x16_t sacc[2], sacc2[2];
      sacc[0] = sacc[1] = sacc2[0] = sacc2[1] = f32x16_t{};
      auto kfrag = [&](int s, int mt) {
        const int r = mt * 32 + lrow;
        return load_bf16x8(Ks + r * M::kLdK + (((2 * s + half) ^ (r & 7)) * 8));
      };
      bf16x8_t kf[3][2];
      kf[0][0] = kfrag(0, 0);
      kf[0][1] = kfrag(0, 1);
      if (M::kKS > 1) {
        kf[1][0] = kfrag(1, 0);
        kf[1][1] = kfrag(1, 1);
      }
#pragma unroll
      for (int s = 0; s < M::kKS; ++s) {
        if (s + 2 < M::kKS) {
          kf[(s + 2) % 3][0] = kfrag(s + 2, 0);
          kf[(s + 2) % 3][1] = kfrag(s + 2, 1);
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          if (s & 1)
            sacc2[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % 3][mt], qf[s], sacc2[mt], 0, 0, 0);
          else
            sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % 3][mt], qf[s], sacc[mt], 0, 0, 0);
        }
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) sacc[mt] += sacc2[mt];
      // ---- mask where some pair is out of the window, the causal order or the sequence
      const bool full = K1 <= Q0 && K0 > Q1 - W && K1 < T;
      if (!full) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = K0 + mt * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
            const bool vis = key <= qr && key > qr - W && key < T;
            sacc[mt][j] = vis ? sacc[mt][j] : -__builtin_inff();
          }
      }
      // ---- online softmax of this row (partner half holds the other 32 keys). O and l are kept
      // relative to a running max m that is raised only when a block's max exceeds it by more
      // than 2^8 (in exp2 units) for some row of the wave: the rescale of the 128 accumulators
      // then happens about once per row instead of every block, and the probabilities stay
      // below 2^8. Numerator and denominator use the same m, so the result does not change.
      float mx = -1e30f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[mt][j]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const bool raise = (mx - m_run) * c > 8.0f;
      if (__any(raise)) {  // wave-uniform
        const float m_new = raise ? mx : m_run;
        const float corr = __builtin_amdgcn_exp2f((m_run - m_new) * c);
        l_run *= corr;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < M::kDT; ++dt)
#pragma unroll
          for (int j = 0; j < 16; ++j) oacc[dt][j] *= corr;
      }
      const float mc = m_run * c;
      float ps = 0.0f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[mt][j], c, -mc));
          sacc[mt][j] = p;
          ps += p;
        }
      ps += __shfl_xor(ps, 32, 64);
      l_run += ps;
      // ---- O^T += V^T P^T over the block's 4 steps of 16 keys. P enters as bf16 hi + lo (two
      // MFMAs on the same V^T fragment): with P in bf16 alone, rows that attend to few keys and
      // whose output cancels (|o| well below its terms) lose ~1e-2 of the output's rms.
      auto vfrag = [&](int s4, int dt) {
        // V^T[d][keys kc..kc+3, kc+8..kc+11] of this half, d = 32 dt + lrow: 2-byte reads of the
        // raw rows (32 lanes on 32 consecutive d of one row per read)
        const int kc = s4 * 16 + 4 * half;
        const unsigned short *col = reinterpret_cast<const unsigned short *>(Vs) + dt * 32 + lrow;
        u32x4_t u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = kc + (e >> 1) * 8 + (e & 1) * 2;
          u[e] = static_cast<uint32_t>(col[key * M::kLdV]) |
                 (static_cast<uint32_t>(col[(key + 1) * M::kLdV]) << 16);
        }
        return __builtin_bit_cast(bf16x8_t, u);
      };
      bf16x8_t vf[2][M::kDT];  // V^T fragments, one 16-key step ahead
#pragma unroll
      for (int dt = 0; dt < M::kDT; ++dt) vf[0][dt] = vfrag(0, dt);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        if (s4 + 1 < 4) {
#pragma unroll
          for (int dt = 0; dt < M::kDT; ++dt) vf[(s4 + 1) & 1][dt] = vfrag(s4 + 1, dt);
        }
        const int mt = s4 >> 1, jb = (s4 & 1) * 8;
        u32x4_t ph, pl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = sacc[mt][jb + 2 * e], p1 = sacc[mt][jb + 2 * e + 1];
          ph[e] = pack_bf16x2(p0, p1);
          pl[e] = pack_bf16x2(p0 - bf16lo(ph[e]), p1 - bf16hi(ph[e]));
        }
        const bf16x8_t pfh = __builtin_bit_cast(bf16x8_t, ph);
        const bf16x8_t pfl = __builtin_bit_cast(bf16x8_t, pl);
#pragma unroll
        for (int dt = 0; dt < M::kDT; ++dt)
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[s4 & 1][dt], pfh, oacc[dt], 0, 0, 0);
#pragma unroll
        for (int dt = 0; dt < M::kDT; ++dt)
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[s4 & 1][dt], pfl, oacc[dt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next block's K rows landed
    __syncthreads();
  }
  // ---- normalise and store: lane = row qr, d = 32 dt + 8 (j / 4) + 4 half + (j % 4)
  if (qr < T) {
    const float inv = 1.0f / l_run;
    bf16_t *op = o + (static_cast<size_t>(b) * T + qr) * qstride + static_cast<size_t>(h) * DH;
#pragma unroll
    for (int dt = 0; dt < M::kDT; ++dt)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d = dt * 32 + 8 * jg + 4 * half;
        const uint2 pk = make_uint2(pack_bf16x2(oacc[dt][4 * jg] * inv, oacc[dt][4 * jg + 1] * inv),
                                    pack_bf16x2(oacc[dt][4 * jg + 2] * inv, oacc[dt][4 * jg + 3] * inv));
        *reinterpret_cast<uint2 *>(op + d) = pk;
      }
  }
}

bool local_mqa_supported(int dh) { return dh == 64 || dh == 128 || dh == 256; }

hipError_t launch_local_mqa(const void *q, const void *k, const void *v, void *o, int B, int T,
                            int Hq, int dh, int window, float scale, hipStream_t s) {
  const float c = scale * 1.4426950408889634f;
  const dim3 grid((T + 127) / 128, Hq, B);
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
