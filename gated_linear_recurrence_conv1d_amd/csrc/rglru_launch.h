// rglru_launch.h -- internal launchers shared between the kernel files and the C ABI layer.
// Every launcher assumes its arguments were validated by the ABI layer (rglru_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace rglru {

enum IoType { kF32 = 0, kBF16 = 1 };

// Bytes of one (pa, px) pre-activation pair in the workspace.
inline size_t pre_pair_bytes(int io) { return io == kBF16 ? 4 : 8; }

// Gate projections: conv + block-diagonal matmuls + biases -> pre[B][T][D] pairs. split (bf16
// MFMA path only): the conv output enters the contraction as bf16 hi + lo instead of bf16.
hipError_t launch_gates(const void *x, const void *conv_w, const void *W_a, const float *b_a,
                        const void *W_x, const float *b_x, void *pre, int B, int T, int D, int H,
                        int io, hipStream_t s, bool split = false);

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

// conv_state[b] = the last three inputs of sequence b (zeros before t = 0).
hipError_t launch_prefill_state(const void *x, void *conv_state, int B, int T, int D, int io,
                                hipStream_t s);

// One decode step for N rows, in place on conv_state and h.
hipError_t launch_decode(const void *x_t, void *conv_state, float *h, void *y_t,
                         const void *conv_w, const void *W_a, const float *b_a, const void *W_x,
                         const float *b_x, const float *Lambda, int N, int D, int H, int io,
                         hipStream_t s);

// Every forward and backward workspace starts with kCtrlBytes of control words: word 1 counts
// the look-back waits that gave up (zero after any call that completed normally), the words
// after it are the fused passes' tile tickets. Calls whose plan has no waits clear word 1 with
// launch_clear_words.
constexpr size_t kCtrlBytes = 256;
hipError_t launch_clear_words(unsigned *p, int n, hipStream_t s);

// Single-pass fused forward (bf16 I/O, Dh in {32, 64, 128, 256}, T * D < 2^31 so that offsets
// within one sequence fit in 32 bits): conv + MFMA gates + gate
// nonlinearity + scan with a decoupled look-back across 64-step time tiles. ctrl_ws:
// fused_ctrl_bytes(H) of control words followed by fused_slots() 64-bit look-back words (one per
// tile and channel); both are reset by the launcher before the main kernel.
bool fused_supported(int io, int T, int D, int Dh);
size_t fused_ctrl_bytes(int H);
size_t fused_slots(int B, int T, int H, int Dh);
hipError_t launch_fused(const void *x, const void *conv_w, const void *W_a, const float *b_a,
                        const void *W_x, const float *b_x, const float *Lambda, const float *h0,
                        void *y, float *h_T, int B, int T, int D, int H, void *ctrl_ws,
                        hipStream_t s);
// The split plan's scan with the same kernel, the gate pre-activations read from pre (fp16
// pairs, biases included) instead of computed (shapes as fused_supported), over groups of
// scan_tiled_group(Dh) channels: ctrl 2 + scan_tiled_groups(D, H) words and fused_slots()
// look-back words, reset by the launcher; gave_up counts look-back waits that gave up (reset by
// the launcher too).
int scan_tiled_group(int Dh);
int scan_tiled_groups(int D, int H);
hipError_t launch_scan_tiled(const void *x, const void *pre, const void *conv_w,
                             const float *Lambda, const float *h0, void *y, float *h_T, int B,
                             int T, int D, int H, unsigned *ctrl, unsigned *gave_up,
                             unsigned long long *words, hipStream_t s);

// The weight contractions as persistent workgroups with resident weights (bf16): gate
// pre-activations (Dh in {32, 64, 128, 256}; split: the conv output as bf16 hi + lo, as the
// backward recomputes them, else as bf16, as the forward plans round it), and the backward's
// dxc += dp [W_a ; W_x] from the interleaved transposed weights wti (Dh in {128, 256}).
// Both need T * D * 4 < 2^31 (32-bit buffer offsets within one sequence).
bool resident_preacts_supported(int Dh);
bool resident_dxc_supported(int Dh);
hipError_t launch_resident_preacts(const void *x, const void *conv_w, const void *W_a,
                                   const float *b_a, const void *W_x, const float *b_x,
                                   void *pre, int B, int T, int D, int H, hipStream_t s,
                                   bool split);
// dxd: the direct part of dxc (fp16, from the per-element pass); writes dx and the dconv_w
// partial sums pcw[B][ceil(T / 64)][4][D] (the conv's transpose fused in).
hipError_t launch_resident_dxc(const void *dp, const void *wti, const uint16_t *dxd,
                               const void *x, const void *conv_w, void *dx, float *pcw, int B,
                               int T, int D, int H, hipStream_t s);

// The backward's per-element part in one pass over kFusedBwdRows-step tiles, latest first (bf16, Dh in
// {128, 256}, T * D * 4 < 2^31): pre-activations recomputed on MFMA, the adjoint carried from
// tile to tile, and dpre (fp16 pairs) / dxc / the per-tile partial sums / dh0 as the separate
// kernels produce them. ctrl: 2 + H words, slots: fused_backward_slots(B, T, D) words (both reset here).
bool fused_backward_supported(int Dh);
size_t fused_backward_slots(int B, int T, int D);
hipError_t launch_fused_backward(const void *x, const void *y, const void *dy, const float *h0,
                                 const float *dh_T, const void *conv_w, const void *W_a,
                                 const float *b_a, const void *W_x, const float *b_x,
                                 const float *Lambda, uint32_t *dpre, uint16_t *dxc,
                                 float *part, float *dh0, int B, int T, int D, int H,
                                 unsigned *ctrl, unsigned long long *slots, hipStream_t s);

// Local sliding-window multi-query attention, forward (bf16, dh in {64, 128, 256}).
bool local_mqa_supported(int dh);
hipError_t launch_local_mqa(const void *q, const void *k, const void *v, void *o, int B, int T,
                            int Hq, int dh, int window, float scale, hipStream_t s);

// Backward (gradients of every input and parameter). Time is cut into chunks of kBwdChunk steps
// for the reverse scan. BwdLayout gives the workspace carve (byte offsets, 256-byte aligned) and
// the row split of the dW contraction; launch_backward assumes a workspace of layout.total bytes.
constexpr int kBwdChunk = 64;
constexpr int kBwdCUs = 256;  // CUs the dW split is sized for (MI355X)
constexpr int kFusedBwdRows = 32;  // tile of the fused per-element pass
struct BwdLayout {
  int nC;                     // chunks per sequence
  int nCp;                    // partial-sum rows per sequence (chunks, or fused-pass tiles)
  int S;                      // row splits of the dW contraction
  int rows_per_split;         // rows of the flattened (b, t) index per split
  bool mfma_dxc, mfma_dw;     // which contractions run on MFMA
  bool fused;                 // the per-element part as one tile pass (no pre, sums, carry)
  size_t o_pre, o_dpre, o_dxc, o_sums, o_carry, o_part, o_pcw, o_pw, o_wti, o_ctrl, o_lb,
      total;
};
BwdLayout backward_layout(int B, int T, int D, int H, int io);
hipError_t launch_backward(const void *x, const void *conv_w, const void *W_a, const float *b_a,
                           const void *W_x, const float *b_x, const float *Lambda,
                           const float *h0, const void *y, const void *dy, const float *dh_T,
                           void *dx, float *dconv_w, float *dW_a, float *db_a, float *dW_x,
                           float *db_x, float *dLambda, float *dh0, int B, int T, int D, int H,
                           int io, void *workspace, hipStream_t s);

}  // namespace rglru
