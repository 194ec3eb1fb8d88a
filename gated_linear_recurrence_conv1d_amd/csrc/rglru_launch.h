// rglru_launch.h -- internal launchers shared between the kernel files and the C ABI layer.
// Every launcher assumes its arguments were validated by the ABI layer (rglru_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace rglru {

enum IoType { kF32 = 0, kBF16 = 1 };

// Bytes of one (pa, px) pre-activation pair in the workspace.
inline size_t pre_pair_bytes(int io) { return io == kBF16 ? 4 : 8; }

// Gate projections: conv + block-diagonal matmuls + biases -> pre[B][T][D] pairs.
hipError_t launch_gates(const void *x, const void *conv_w, const void *W_a, const float *b_a,
                        const void *W_x, const float *b_x, void *pre, int B, int T, int D, int H,
                        int io, hipStream_t s);

// Direct scan: one lane per (b, d) over all T steps.
hipError_t launch_scan_direct(const void *x, const void *pre, const void *conv_w,
                              const float *Lambda, const float *h0, void *y, float *h_T, int B,
                              int T, int D, int io, hipStream_t s);

// Chunked scan in three passes with chunk length L. sums: [B][nC][D] float2 (sum of log a,
// local end state); carry: [B][nC][D] float (state entering each chunk).
hipError_t launch_scan_chunked(const void *x, const void *pre, const void *conv_w,
                               const float *Lambda, const float *h0, void *y, float *h_T, int B,
                               int T, int D, int L, float2 *sums, float *carry, int io,
                               hipStream_t s);

// One decode step for N rows, in place on conv_state and h.
hipError_t launch_decode(const void *x_t, void *conv_state, float *h, void *y_t,
                         const void *conv_w, const void *W_a, const float *b_a, const void *W_x,
                         const float *b_x, const float *Lambda, int N, int D, int H, int io,
                         hipStream_t s);

// Single-pass fused forward (bf16 I/O, Dh in {32, 64, 128, 256}, T * D < 2^31 so that offsets
// within one sequence fit in 32 bits): conv + MFMA gates + gate
// nonlinearity + scan with a decoupled look-back across 64-step time tiles. ctrl_ws:
// fused_ctrl_bytes(H) of control words followed by 2 * fused_slots() 64-bit look-back words;
// both are reset by the launcher before the main kernel.
bool fused_supported(int io, int T, int D, int Dh);
size_t fused_ctrl_bytes(int H);
size_t fused_slots(int B, int T, int H, int Dh);
hipError_t launch_fused(const void *x, const void *conv_w, const void *W_a, const float *b_a,
                        const void *W_x, const float *b_x, const float *Lambda, const float *h0,
                        void *y, float *h_T, int B, int T, int D, int H, void *ctrl_ws,
                        hipStream_t s);

}  // namespace rglru
