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
// contraction needs. K is staged row-major with rows padded by 16 bytes, V transposed (row d holds
// the block's 64 keys, padded to 136 bytes), both double buffered: block j+1 is loaded into
// registers before block j's MFMAs and written to the other buffer after them.
#include "rglru_launch.h"
#include "rglru_mfma.h"

namespace rglru {

template <int DH> struct Mqa {
  static_assert(DH == 64 || DH == 128 || DH == 256, "local MQA tile needs dh in {64, 128, 256}");
  static constexpr int kQB = 128;               // query rows per workgroup
  static constexpr int kKB = 64;                // keys per block
  static constexpr int kThreads = 256;          // 4 waves x 32 rows
  static constexpr int kKS = DH / 16;           // k-steps of S^T = K Q^T
  static constexpr int kDT = DH / 32;           // 32-row d tiles of O^T
  static constexpr int kLdK = DH + 8;           // bf16 per K row
  static constexpr int kLdV = kKB + 4;          // bf16 per V^T row (136 bytes)
  static constexpr int kKElems = kKB * kLdK;
  static constexpr int kVElems = DH * kLdV;
  static constexpr int kBuf = kKElems + kVElems;
  static constexpr int kKChunks = kKB * DH / 8 / kThreads;    // 16-byte K pieces per thread
  static constexpr int kVTotal = (kKB / 4) * (DH / 8);          // items of 4 keys x 8 d
  static constexpr int kVItems = (kVTotal + kThreads - 1) / kThreads;
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

  // ---- staging: K pieces (row, 16 B) and V items (4 keys x 8 d), through registers
  u32x4_t kr[M::kKChunks];
  u32x4_t vr[M::kVItems][4];
  auto load_block = [&](int kb) {
    const int key0 = kb * M::kKB;
#pragma unroll
    for (int i = 0; i < M::kKChunks; ++i) {
      const int cidx = tid + i * M::kThreads;
      const int row = cidx / (DH / 8), col = cidx % (DH / 8);
      const int key = key0 + row;
      kr[i] = key < T ? *reinterpret_cast<const u32x4_t *>(kb_ + static_cast<size_t>(key) * DH + col * 8)
                      : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < M::kVItems; ++i) {
      const int it = tid + i * M::kThreads;
      const int kq = it % (M::kKB / 4), doct = it / (M::kKB / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + 4 * kq + r;
        vr[i][r] = (it < M::kVTotal && key < T)
                       ? *reinterpret_cast<const u32x4_t *>(vb_ + static_cast<size_t>(key) * DH + doct * 8)
                       : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_block = [&](int buf) {
    bf16_t *Ks = lds + buf * M::kBuf;
    bf16_t *Vt = Ks + M::kKElems;
#pragma unroll
    for (int i = 0; i < M::kKChunks; ++i) {
      const int cidx = tid + i * M::kThreads;
      const int row = cidx / (DH / 8), col = cidx % (DH / 8);
      *reinterpret_cast<u32x4_t *>(Ks + row * M::kLdK + col * 8) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < M::kVItems; ++i) {
      const int it = tid + i * M::kThreads;
      if (it >= M::kVTotal) continue;
      const int kq = it % (M::kKB / 4), doct = it / (M::kKB / 4);
      // V^T[d][4 kq .. 4 kq + 3] for the 8 d of this item: halves of the 4 rows' words
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wd = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t k01 = __builtin_amdgcn_perm(vr[i][1][wd], vr[i][0][wd], sel);
        const uint32_t k23 = __builtin_amdgcn_perm(vr[i][3][wd], vr[i][2][wd], sel);
        *reinterpret_cast<uint2 *>(Vt + (doct * 8 + e) * M::kLdV + 4 * kq) = make_uint2(k01, k23);
      }
    }
  };

  f32x16_t oacc[M::kDT];
#pragma unroll
  for (int dt = 0; dt < M::kDT; ++dt) oacc[dt] = f32x16_t{};
  float m_run = -1e30f, l_run = 0.0f;  // finite start: fully masked blocks give p = 0, corr = 1

  load_block(kb_first);
  store_block(0);
  __syncthreads();
  for (int kb = kb_first; kb <= kb_last; ++kb) {
    const int buf = (kb - kb_first) & 1;
    const bool more = kb < kb_last;
    if (more) load_block(kb + 1);
    const int K0 = kb * M::kKB, K1 = K0 + M::kKB - 1;
    const int Q0 = qw, Q1 = qw + 31;
    // does any (key, row) pair of this wave see each other in this block?
    if (K0 <= Q1 && K1 > Q0 - W && Q0 < T) {
      const bf16_t *Ks = lds + buf * M::kBuf;
      const bf16_t *Vt = Ks + M::kKElems;
      // ---- S^T = K Q^T: 64 keys x 32 rows
      f32x16_t sacc[2];
      sacc[0] = sacc[1] = f32x16_t{};
#pragma unroll
      for (int s = 0; s < M::kKS; ++s)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8_t af = load_bf16x8(Ks + (mt * 32 + lrow) * M::kLdK + s * 16 + half * 8);
          sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[s], sacc[mt], 0, 0, 0);
        }
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
      // ---- online softmax of this row (partner half holds the other 32 keys)
      float mx = -1e30f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[mt][j]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float corr = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      const float mc = m_new * c;
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
      l_run = fmaf(l_run, corr, ps);
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < M::kDT; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[dt][j] *= corr;
      // ---- O^T += V^T P^T over the block's 4 steps of 16 keys. P enters as bf16 hi + lo (two
      // MFMAs on the same V^T fragment): with P in bf16 alone, rows that attend to few keys and
      // whose output cancels (|o| well below its terms) lose ~1e-2 of the output's rms.
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
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
        const int kc = s4 * 16 + 4 * half;  // this half's keys kc..kc+3 and kc+8..kc+11
        bf16x8_t af[M::kDT];
#pragma unroll
        for (int dt = 0; dt < M::kDT; ++dt) {
          const bf16_t *row = Vt + (dt * 32 + lrow) * M::kLdV;
          af[dt] = lds_read_4x2(row + kc, row + kc + 8);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[dt], pfh, oacc[dt], 0, 0, 0);
        }
#pragma unroll
        for (int dt = 0; dt < M::kDT; ++dt)
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[dt], pfl, oacc[dt], 0, 0, 0);
      }
    }
    if (more) store_block(buf ^ 1);
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
