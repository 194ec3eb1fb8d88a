// rglru_device.h -- device-side element types and the RG-LRU gate math for gfx950.
//
// The gate math follows the RG-LRU as this library defines it (the Griffin paper page on
// docshare.wps.com names the layer in its abstract and Introduction but prints no equations; the
// recurrence gate that can drop the input and keep the history is the one of Soham De's Griffin
// thread, tweet on adding a Recurrent Gate to LRU):
//   r = sigmoid(pa), i = sigmoid(px), log a = -8 r softplus(-Lambda),
//   a = exp(log a), m = sqrt(1 - a^2), u = m * i * xc, h <- a h + u.
// In fp32, 1 - a*a cancels catastrophically when a is near 1 (a^8 = 0.9999 and r = 0.01 give
// 1 - a^2 ~ 2e-6, where the literal form loses about 1e-2 of relative accuracy). So both a and
// 1 - a^2 come from one e = expm1(log a): a = 1 + e and 1 - a^2 = -e (2 + e), which is exact
// algebra and keeps full relative accuracy. On [-1/4, 0], expm1(z) = z q(z) with q the degree-4
// polynomial interpolating expm1(z)/z at the five Chebyshev nodes of that interval (relative
// error below 2.7e-9 before fp32 rounding, so the fp32 evaluation is good to about 1e-7); below
// -1/4 it is exp(z) - 1, whose cancellation costs at most a few ulps because |e| > 0.22.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rglru {

constexpr int kConvW = 4;      // temporal conv width
constexpr float kGateC = 8.0f;  // the fixed scale c of the recurrence gate

typedef uint16_t bf16_t;  // raw bf16 bits

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// fp32 -> bf16 with round-to-nearest-even (gfx950 converts in hardware, v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  const bf16x2_v v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// (pa, px) pre-activation pair for the bf16 path: two fp16 values (round-to-nearest-even),
// pa in the low half. fp16 keeps 11 significant bits; values beyond its range become +-inf,
// which the sigmoids map to exactly 0 or 1, as the exact values would be after rounding.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  _Float16 a = static_cast<_Float16>(lo);
  _Float16 b = static_cast<_Float16>(hi);
  uint16_t ua, ub;
  __builtin_memcpy(&ua, &a, 2);
  __builtin_memcpy(&ub, &b, 2);
  return static_cast<uint32_t>(ua) | (static_cast<uint32_t>(ub) << 16);
}
__device__ __forceinline__ float f16lo(uint32_t v) {
  uint16_t u = static_cast<uint16_t>(v & 0xffffu);
  _Float16 h;
  __builtin_memcpy(&h, &u, 2);
  return static_cast<float>(h);
}
__device__ __forceinline__ float f16hi(uint32_t v) {
  uint16_t u = static_cast<uint16_t>(v >> 16);
  _Float16 h;
  __builtin_memcpy(&h, &u, 2);
  return static_cast<float>(h);
}

// Element I/O traits: float or bf16 storage, fp32 arithmetic.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float *p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float *p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t *p, size_t i) {
    return bf16_to_f32(p[i]);
  }
  __device__ __forceinline__ static void store(bf16_t *p, size_t i, float v) {
    p[i] = f32_to_bf16(v);
  }
};

// Pre-activation pair storage: float2 for fp32 I/O, fp16x2 in a uint32 for bf16 I/O.
template <typename T> struct PrePair;
template <> struct PrePair<float> {
  typedef float2 type;
  __device__ __forceinline__ static type pack(float pa, float px) { return make_float2(pa, px); }
  __device__ __forceinline__ static float pa(type v) { return v.x; }
  __device__ __forceinline__ static float px(type v) { return v.y; }
};
template <> struct PrePair<bf16_t> {
  typedef uint32_t type;
  __device__ __forceinline__ static type pack(float pa, float px) { return pack_f16x2(pa, px); }
  __device__ __forceinline__ static float pa(type v) { return f16lo(v); }
  __device__ __forceinline__ static float px(type v) { return f16hi(v); }
};

constexpr float kLog2e = 1.4426950408889634f;

// Words of a tile-to-tile look-back (a carried state crossing 64-step tiles of one sequence):
// two fp32 in one 64-bit word, stored and loaded as single relaxed agent-scope atomics (each word
// is self-contained, so no release/acquire fences are needed). kEmpty marks a word not yet
// written (a NaN pattern no pack2 produces: pack2 canonicalises NaN in its low half); waits are
// bounded by kMaxSpin polls, after which the waiting tile writes NaN instead of hanging.
constexpr unsigned long long kEmpty = ~0ull;
constexpr unsigned kMaxSpin = 1u << 26;
// A word that carries either a tile's aggregate (A, U) = pack2(A, U) or, later, its inclusive
// state h: kInclTag in the low half (a NaN payload that pack2 never produces, since it
// canonicalises NaN to 0x7FC00000, and that differs from kEmpty's) and h in the high half.
constexpr uint32_t kInclTag = 0x7FC00001u;
__device__ __forceinline__ unsigned long long pack_incl(float h) {
  return static_cast<unsigned long long>(kInclTag) |
         (static_cast<unsigned long long>(__float_as_uint(h)) << 32);
}
__device__ __forceinline__ bool is_incl(unsigned long long v) {
  return static_cast<uint32_t>(v) == kInclTag;
}

// Body of the look-back resets: n words (16-byte aligned) to kEmpty with one 16-byte store per
// lane and step, and nctrl control words to 0 (block 0).
__device__ __forceinline__ void fill_lookback(unsigned long long *slots, size_t n, unsigned *ctrl,
                                              int nctrl) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  ulonglong2 *s2 = reinterpret_cast<ulonglong2 *>(slots);
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n / 2;
       i += stride)
    s2[i] = make_ulonglong2(kEmpty, kEmpty);
  if (blockIdx.x == 0) {
    if (threadIdx.x == 0 && (n & 1)) slots[n - 1] = kEmpty;
    for (int i = threadIdx.x; i < nctrl; i += blockDim.x) ctrl[i] = 0u;
  }
}
// Blocks of 256 threads for a fill of n words.
inline unsigned fill_blocks(size_t n) {
  const size_t b = (n / 2 + 255) / 256;
  return static_cast<unsigned>(b < 1 ? 1 : (b > 8192 ? 8192 : b));
}
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

// Byte count or offset of n rows of D elements of `bytes` bytes, in unsigned 32-bit arithmetic:
// callers keep every such value below 2^32 (the buffer descriptors' range), and a negative row
// (the conv halo before t = 0) wraps past the end of the buffer, as the range check needs.
__device__ __forceinline__ unsigned row_bytes(int rows, int D, unsigned bytes) {
  return static_cast<unsigned>(rows) * static_cast<unsigned>(D) * bytes;
}
// The same as the int the buffer-descriptor builtin takes for its record count.
__device__ __forceinline__ int rec_bytes(int T, int D, unsigned bytes) {
  return __builtin_bit_cast(int, row_bytes(T, D, bytes));
}

// One 16-byte-per-lane buffer load straight into LDS (the wave's 64 lanes fill 1 KB from byte
// lds_base on), written as inline asm: for the builtin form the compiler cannot tell which LDS
// bytes the load writes, so it makes later LDS reads -- and every __syncthreads -- wait for all of
// the wave's outstanding vector memory operations. Kernels that use it order the loads
// themselves (s_waitcnt vmcnt, then a barrier, before any wave reads the rows; a barrier before
// a buffer is refilled). M0 (the LDS base) is restored afterwards.
__device__ __forceinline__ void dma_16b(__amdgpu_buffer_rsrc_t rsrc, unsigned voff,
                                        unsigned lds_base) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(lds_base), "s"(rsrc));
}

// LDS byte address of a __shared__ pointer (the low half of its generic address), wave-uniform.
__device__ __forceinline__ unsigned lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane(static_cast<unsigned>(reinterpret_cast<uintptr_t>(p)));
}

// Both halves' values of v in every lane: lo from lane (l & 31), hi from lane (l | 32).
// v_permlane32_swap exchanges lanes 32..63 of its first operand with lanes 0..31 of its second;
// with both operands holding v, the first then holds the low half twice and the second the high.
__device__ __forceinline__ void halves(float v, float &lo, float &hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// p, the same in every lane, read from the first one, so that the compiler keeps it (and a buffer
// descriptor made from it) in scalar registers: where it cannot prove a value uniform (64-bit
// offset arithmetic runs on the vector ALU; values that cross a lambda or a divergent loop), a
// descriptor in vector registers wraps every access in a loop over its distinct values, and an
// inline-asm operand that needs scalar registers does not assemble.
template <typename P> __device__ __forceinline__ P *wave_uniform(P *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<P *>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads it does not wait for the
// wave's outstanding vector memory loads and stores, so they stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Per-channel constant kd = -c * softplus(-Lambda), so that log a = kd * r. softplus is taken
// as max(z,0) + log1p(exp(-|z|)); computed once per lane with the accurate library functions.
__device__ __forceinline__ float decay_coeff(float lambda) {
  float z = -lambda;
  float sp = fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z)));
  return -kGateC * sp;
}

// 1 / (1 + exp(-v)) with the hardware exp2 and reciprocal. v = -inf.. : exp2 overflows to inf and
// the reciprocal returns exactly 0; large positive v gives exp2 = 0 and exactly 1.
__device__ __forceinline__ float fast_sigmoid(float v) {
  float e = __builtin_amdgcn_exp2f(-v * kLog2e);
  return __builtin_amdgcn_rcpf(1.0f + e);
}

// expm1 on [-1/4, 0] as z q(z), q the Chebyshev interpolant of expm1(z)/z (see the header
// comment); coefficients of q from degree 0 to 4.
constexpr float kExpm1Q0 = 1.0f;
constexpr float kExpm1Q1 = 4.999995232e-01f;
constexpr float kExpm1Q2 = 1.666510850e-01f;
constexpr float kExpm1Q3 = 4.149065539e-02f;
constexpr float kExpm1Q4 = 7.513605990e-03f;
__device__ __forceinline__ float expm1_poly(float z) {
  float p = fmaf(z, kExpm1Q4, kExpm1Q3);
  p = fmaf(z, p, kExpm1Q2);
  p = fmaf(z, p, kExpm1Q1);
  p = fmaf(z, p, kExpm1Q0);
  return z * p;
}

// expm1(z) for z <= 0 (log a is never positive).
__device__ __forceinline__ float expm1_nonpos(float z) {
  float e = expm1_poly(z);
  if (z < -0.25f) e = __builtin_amdgcn_exp2f(z * kLog2e) - 1.0f;
  return e;
}

// One RG-LRU gate evaluation: returns the decay a and the gated, normalised input u.
__device__ __forceinline__ void gate(float pa, float px, float xc, float kd, float &a, float &u) {
  float r = fast_sigmoid(pa);
  float ig = fast_sigmoid(px);
  float e = expm1_nonpos(kd * r);
  a = 1.0f + e;
  float w = -e * (2.0f + e);  // 1 - a^2, >= 0
  float m = __builtin_amdgcn_sqrtf(w);
  u = m * (ig * xc);
}

}  // namespace rglru
