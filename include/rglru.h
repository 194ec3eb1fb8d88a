/*
 * rglru.h -- C ABI of the MI355X (gfx950) library for Griffin's recurrent-block hot path:
 * a causal depthwise temporal Conv1D of width 4 feeding the RG-LRU gated linear recurrence.
 *
 * What is computed (per batch b, channel d, time t; head g = d / Dh, o = d % Dh):
 *   xc[t][d] = sum_{j=0..3} conv_w[j][d] * x[t-3+j][d]        x before t = 0 reads zero
 *   pa = b_a[d] + sum_i W_a[g][o][i] * xc[t][g*Dh+i]          block-diagonal gates, out = W in
 *   px = b_x[d] + sum_i W_x[g][o][i] * xc[t][g*Dh+i]
 *   r = sigmoid(pa), i = sigmoid(px), log a = -8 * r * softplus(-Lambda[d])
 *   h[t] = a * h[t-1] + sqrt(1 - a^2) * (i * xc[t]);   y[t] = h[t]
 * Sources: the temporal Conv1D in the recurrent block and the recurrence gate that can drop the
 * input at time t and keep the history (Soham De's Griffin thread, muskviewer.com, the tweets on
 * keeping the recurrent block simple and on adding a Recurrent Gate to LRU); gates that do not
 * read the recurrent state and a fixed-size state (alby13 blog "Beyond Transformer Architecture:
 * Griffin and Google RecurrentGemma", section "Core Components of Griffin -- 1. RG-LRU"); the
 * diagonal recurrence (Soham De's thread, tweet on S4D/LRU); the RG-LRU layer itself is named by
 * the Griffin paper page on docshare.wps.com (abstract and Introduction). The pages print no
 * equations: the ones above are the RG-LRU's as this library defines it, c = 8.
 *
 * Conventions for every entry point:
 *  - Pointers named x, y, conv_w, W_a, W_x, conv_state, workspace, b_a, b_x, Lambda, h0, h_T, h
 *    are DEVICE pointers (hipMalloc'd or torch CUDA tensors on the current device), contiguous,
 *    row-major, 16-byte aligned. The caller owns all memory; the library never allocates or
 *    frees and keeps no state between calls, so calls on different streams with different
 *    workspaces may run concurrently.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream. Execution is
 *    asynchronous on that stream; the status reflects argument checks and launch errors only.
 *  - Argument checks happen before any launch; a failed check launches nothing.
 *  - dtype selects the element type of x, y, conv_w, W_a, W_x and conv_state (fp32 or bf16).
 *    b_a, b_x, Lambda, h0, h_T and h are always fp32.
 *  - Supported sizes: B, T, D, H, N >= 1; D % H == 0; Dh = D / H <= 256. bf16 with Dh in
 *    {32, 64, 128, 256} runs the gate projections on MFMA; other shapes run them on the vector
 *    ALU.
 */
#ifndef RGLRU_H
#define RGLRU_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RGLRU_OK = 0,
  RGLRU_ERR_INVALID_ARG = 1, /* null required pointer, bad size, aliasing output */
  RGLRU_ERR_UNSUPPORTED = 2, /* dtype or Dh outside the supported set */
  RGLRU_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the size query returned */
  RGLRU_ERR_HIP = 4          /* a HIP launch reported an error */
} rglru_status;

typedef enum { RGLRU_F32 = 0, RGLRU_BF16 = 1 } rglru_dtype;

/* How the forward is executed. DIRECT and CHUNKED first write the gate pre-activations to the
 * workspace (MFMA gate projection), then scan: DIRECT has one lane per (b, d) walk all T steps;
 * CHUNKED cuts time into chunks, pass 1 reduces each chunk to (sum of log a, local state), pass 2
 * prefixes those summaries across chunks with a wavefront scan, pass 3 re-scans each chunk from
 * its carry-in; with 64-step chunks on the shapes FUSED takes it runs as one pass instead, the
 * chunks linked by FUSED's decoupled look-back with the pre-activations read rather than
 * computed. FUSED (bf16, Dh in {32, 64, 128, 256}) does everything in one pass over 64-step
 * tiles -- conv, MFMA gates, nonlinearity, in-tile scan -- and links the tiles of a sequence by a
 * decoupled look-back, so HBM sees x once and y once. All give the same result up to fp32
 * rounding and the rounding of stored pre-activations (the scan is associative). DIRECT and the
 * three-pass CHUNKED are bitwise deterministic; FUSED and the one-pass CHUNKED combine whichever
 * predecessor tiles have published when they look back, so their carried state is reproducible
 * to fp32 rounding only. AUTO picks FUSED when supported, else DIRECT or CHUNKED by the number of
 * channels. */
typedef enum {
  RGLRU_PLAN_AUTO = 0,
  RGLRU_PLAN_DIRECT = 1,
  RGLRU_PLAN_CHUNKED = 2,
  RGLRU_PLAN_FUSED = 3
} rglru_plan;

/* Text for a status code (static storage, never NULL). */
const char *rglru_status_string(rglru_status s);

/* Bytes of device workspace rglru_forward needs for this shape, for any plan. Returns 0 when
 * the shape is invalid. */
size_t rglru_forward_workspace_size(int B, int T, int D, int H, rglru_dtype dt);

/* Bytes of device workspace rglru_forward_planned needs with this plan and chunk length (the
 * smallest workspace that call accepts; rglru_forward_workspace_size covers every plan with
 * chunks of 16 steps or more). Returns 0 when the shape, plan or chunk length is invalid or the
 * plan is unsupported for the shape. */
size_t rglru_forward_workspace_size_planned(int B, int T, int D, int H, rglru_dtype dt,
                                            rglru_plan plan, int chunk_len);

/* Every rglru_forward / rglru_forward_planned / rglru_backward workspace begins with a control
 * block; its failure count is the number of look-back waits of the last such call on this
 * workspace that gave up. The FUSED forward, the one-pass CHUNKED scan and the backward's tile
 * pass link time tiles by bounded waits on words other tiles publish; a wait that exceeds its bound (which only a broken
 * ordering invariant can cause) stops, writes NaN for its channel and bumps the count, so a
 * defect shows as NaN and a nonzero count, never as a hang. Plans without waits set the count to
 * zero. This call waits for `stream` (the copy is ordered after the work queued on it), then
 * writes the count to *count (host memory). workspace_bytes must be at least 256.
 * Returns RGLRU_OK, RGLRU_ERR_INVALID_ARG or RGLRU_ERR_HIP. */
rglru_status rglru_lookback_failures(const void *workspace, size_t workspace_bytes,
                                     unsigned *count, void *stream);

/* The plan and chunk length RGLRU_PLAN_AUTO picks for this shape (host-side query, no launch).
 * Writes *plan (RGLRU_PLAN_DIRECT, _CHUNKED or _FUSED) and *chunk_len (T for DIRECT, the tile
 * length 64 for FUSED). */
rglru_status rglru_forward_plan_info(int B, int T, int D, int H, rglru_dtype dt, int *plan,
                                     int *chunk_len);

/* Full-sequence forward.
 *  x       [B][T][D] dtype          input sequence (channels contiguous)
 *  conv_w  [4][D]    dtype          temporal conv taps; conv_w[3] multiplies the current token
 *  W_a     [H][Dh][Dh] dtype        recurrence-gate weights per head, [out][in]
 *  b_a     [D] f32                  recurrence-gate bias
 *  W_x     [H][Dh][Dh] dtype        input-gate weights per head, [out][in]
 *  b_x     [D] f32                  input-gate bias
 *  Lambda  [D] f32                  decay parameter (a = sigmoid(Lambda)^(8 r))
 *  h0      [B][D] f32 or NULL       initial state (NULL: zeros)
 *  y       [B][T][D] dtype, out     states h[t] rounded to dtype (round-to-nearest-even);
 *                                   must not overlap x or the workspace
 *  h_T     [B][D] f32 or NULL, out  final fp32 state
 *  workspace / workspace_bytes      device scratch of at least rglru_forward_workspace_size()
 * Returns RGLRU_OK or an error code; see the conventions above. */
rglru_status rglru_forward(const void *x, const void *conv_w, const void *W_a, const float *b_a,
                           const void *W_x, const float *b_x, const float *Lambda,
                           const float *h0, void *y, float *h_T, int B, int T, int D, int H,
                           rglru_dtype dt, void *workspace, size_t workspace_bytes,
                           void *stream);

/* rglru_forward with an explicit plan. chunk_len is used by RGLRU_PLAN_CHUNKED (0 = automatic,
 * otherwise 1 <= chunk_len); it is ignored by the other plans. RGLRU_PLAN_FUSED on an
 * unsupported dtype / head size returns RGLRU_ERR_UNSUPPORTED. */
rglru_status rglru_forward_planned(const void *x, const void *conv_w, const void *W_a,
                                   const float *b_a, const void *W_x, const float *b_x,
                                   const float *Lambda, const float *h0, void *y, float *h_T,
                                   int B, int T, int D, int H, rglru_dtype dt, void *workspace,
                                   size_t workspace_bytes, void *stream, rglru_plan plan,
                                   int chunk_len);

/* rglru_forward for callers that cannot allocate device memory -- code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc: the same plans and kernels as
 * rglru_forward (automatic plan), with no workspace argument. The workspace is a fixed array the
 * library owns, rglru_forward_noalloc_max_bytes() = 72 MiB on each GPU it runs on (held until the
 * process ends); its device address is looked up once per device, on that device's first call.
 * The call allocates nothing. Shapes whose automatic plan needs more workspace than the array
 * holds return RGLRU_ERR_UNSUPPORTED before any launch (the fused plan needs about B*T*D/8 bytes:
 * up to 600M elements fit). All calls on one GPU share its array: calls that overlap in time on
 * one GPU (other streams, other threads) race and must be serialised by the caller. Arguments,
 * layouts, checks and other errors as for rglru_forward; RGLRU_ERR_HIP if the array cannot be
 * located on the current device. */
rglru_status rglru_forward_noalloc(const void *x, const void *conv_w, const void *W_a,
                                   const float *b_a, const void *W_x, const float *b_x,
                                   const float *Lambda, const float *h0, void *y, float *h_T,
                                   int B, int T, int D, int H, rglru_dtype dt, void *stream);
size_t rglru_forward_noalloc_max_bytes(void);

/* The gate projections alone (conv + block-diagonal matmuls + biases), as the forward computes
 * them before its scan. pre [B][T][D] holds one (pa, px) pair per element: two fp16 values
 * (pa in the low half) for bf16, two fp32 values (pa first) for fp32. */
rglru_status rglru_gate_preacts(const void *x, const void *conv_w, const void *W_a,
                                const float *b_a, const void *W_x, const float *b_x, void *pre,
                                int B, int T, int D, int H, rglru_dtype dt, void *stream);

/* Bytes of device workspace rglru_scan_preacts needs for this shape, for any plan with chunk
 * length >= 16 (0 when the shape is invalid). */
size_t rglru_scan_workspace_size(int B, int T, int D, int H, rglru_dtype dt);

/* The scan stage alone: conv recomputed from x, gate nonlinearity and RG-LRU scan, reading the
 * pre-activation pairs in the layout rglru_gate_preacts writes. Arguments as for
 * rglru_forward_planned (plan AUTO, DIRECT or CHUNKED; FUSED is rejected as invalid, it has no
 * separate scan stage); `pre` must not overlap y; workspace holds only the chunk summaries, or
 * for the one-pass CHUNKED form the look-back words and tickets (RGLRU_PLAN_DIRECT needs none:
 * workspace may then be NULL). rglru_forward with the DIRECT or
 * CHUNKED plan is exactly rglru_gate_preacts followed by this call. */
rglru_status rglru_scan_preacts(const void *x, const void *pre, const void *conv_w,
                                const float *Lambda, const float *h0, void *y, float *h_T, int B,
                                int T, int D, int H, rglru_dtype dt, void *workspace,
                                size_t workspace_bytes, void *stream, rglru_plan plan,
                                int chunk_len);

/* One decode step for N independent sequences, in place: the same conv, gates and recurrence for
 * T = 1, continuing from a fixed-size per-sequence state -- the last three inputs and the fp32 h
 * -- which is what makes the recurrent model's decoding fast and its memory constant (alby13
 * blog "Beyond Transformer Architecture: Griffin and Google RecurrentGemma", sections "Core
 * Components of Griffin -- 1. RG-LRU" and "Griffin's Strengths").
 *  x_t         [N][D] dtype                new token per row
 *  conv_state  [N][3][D] dtype, in/out     last three inputs, oldest first; becomes
 *                                          (cs[1], cs[2], x_t)
 *  h           [N][D] f32, in/out          recurrent state
 *  y_t         [N][D] dtype, out           new state rounded to dtype; must not overlap the
 *                                          other buffers
 *  conv_w, W_a, b_a, W_x, b_x, Lambda      as for rglru_forward
 * Returns RGLRU_OK or an error code. */
rglru_status rglru_decode_step(const void *x_t, void *conv_state, float *h, void *y_t,
                               const void *conv_w, const void *W_a, const float *b_a,
                               const void *W_x, const float *b_x, const float *Lambda, int N,
                               int D, int H, rglru_dtype dt, void *stream);

/* Prefill -> decode hand-off. After rglru_forward over x (which returns the final state h_T), this
 * writes the conv state that rglru_decode_step continues from: conv_state[b][j] = x[b][T-3+j]
 * for j = 0..2 (oldest first), zero where T-3+j < 0 -- the inputs the conv sees before the next
 * step, with the forward's zero padding before t = 0. With h = h_T, decode steps on the
 * following tokens then continue the sequence exactly as a forward over the concatenation would
 * (the fixed-size state that makes decoding fast: alby13 blog, "Core Components of Griffin -- 1.
 * RG-LRU" and "Griffin's Strengths").
 *  x           [B][T][D] dtype       the prefilled inputs
 *  conv_state  [B][3][D] dtype, out  must not overlap x
 * Returns RGLRU_OK or an error code. */
rglru_status rglru_prefill_state(const void *x, void *conv_state, int B, int T, int D,
                                 rglru_dtype dt, void *stream);

/* Local (sliding-window) multi-query attention, forward: Griffin's other temporal-mixing block,
 * whose query heads share one key/value head and whose positions attend only within a fixed
 * window of recent positions, typically 1024 (alby13 blog "Beyond Transformer Architecture: Griffin
 * and Google RecurrentGemma", section "Core Components of Griffin -- 2. Local Sliding-Window MQA";
 * Soham De's Griffin thread, tweet on adding a local attention block every two recurrent blocks).
 *   o[b][t][h] = sum_u softmax_u(scale * <q[b][t][h], k[b][u]>) v[b][u],
 *   u in [max(0, t - window + 1), t]   (the window holds `window` positions including t).
 *  q  [B][T][Hq][dh] bf16    query heads
 *  k  [B][T][dh] bf16        the shared key head
 *  v  [B][T][dh] bf16        the shared value head
 *  o  [B][T][Hq][dh] bf16, out, must not overlap q, k or v
 *  window >= 1; scale > 0, or 0 for 1/sqrt(dh)
 * Softmax and both contractions accumulate in fp32 (MFMA); probabilities enter the second
 * contraction as bf16 hi + lo (about 16 bits). Supported: dt = RGLRU_BF16, dh in {64, 128, 256},
 * T * dh * 2 <= 2^30 bytes per sequence of k (else RGLRU_ERR_UNSUPPORTED). No workspace. */
rglru_status rglru_local_mqa(const void *q, const void *k, const void *v, void *o, int B, int T,
                             int Hq, int dh, int window, float scale, rglru_dtype dt,
                             void *stream);

/* Bytes of device workspace rglru_backward needs for this shape (0 when the shape is invalid).
 * About 4 B (bf16) or 8 B (fp32) of pre-activations, the same again of gate gradients and 4 B of
 * conv-output gradient per element of x, plus chunk summaries and partial sums. */
size_t rglru_backward_workspace_size(int B, int T, int D, int H, rglru_dtype dt);

/* Gradients of a scalar loss L through rglru_forward, given dL/dy and dL/dh_T. The forward is
 * differentiated exactly (chain rule through the conv, the gate projections, the log-space gates
 * and the scan); the pages print no backward -- they place the method's memory-bound cost in
 * training (Soham De's Griffin thread, muskviewer.com, the tweet on the Pallas kernel and HBM
 * accesses), and the forward it differentiates is the one described above. The reverse-time
 * adjoint delta_t = dy_t + a_{t+1} delta_{t+1} is scanned in time tiles (32 steps in the bf16
 * tile pass for Dh 128 / 256, chunks of 64 steps otherwise) linked across tiles, so the pass has
 * parallelism over time as well as over (b, d).
 *  x, conv_w, W_a, b_a, W_x, b_x, Lambda, h0   the forward's inputs (h0 NULL: zeros)
 *  y       [B][T][D] dtype            the forward's output for these inputs; h[t-1] is read from
 *                                     it (rounded to dtype, like the stored activations of any
 *                                     training step)
 *  dy      [B][T][D] dtype            dL/dy
 *  dh_T    [B][D] f32 or NULL         dL/dh_T (NULL: zeros)
 *  dx      [B][T][D] dtype, out       dL/dx, rounded to dtype
 *  dconv_w [4][D] f32, out            dL/dconv_w
 *  dW_a, dW_x [H][Dh][Dh] f32, out    dL/dW ([out][in], as the weights)
 *  db_a, db_x, dLambda [D] f32, out
 *  dh0     [B][D] f32 or NULL, out    dL/dh0 (written when not NULL, also when h0 is NULL)
 *  workspace / workspace_bytes        at least rglru_backward_workspace_size(); contents on entry
 *                                     are ignored
 * Parameter gradients are fp32 whatever dtype is: each is a sum over all B*T rows. The gate
 * contractions run on bf16 MFMA with fp32 accumulation for bf16 with Dh in {32, 64, 128, 256}
 * (dW on MFMA for Dh in {128, 256}), on the fp32 vector ALU otherwise. Every sum over rows is taken
 * in a fixed order (no floating-point atomics), so results are bitwise reproducible. Outputs must
 * not overlap the inputs, the workspace or each other (RGLRU_ERR_INVALID_ARG). */
rglru_status rglru_backward(const void *x, const void *conv_w, const void *W_a, const float *b_a,
                            const void *W_x, const float *b_x, const float *Lambda,
                            const float *h0, const void *y, const void *dy, const float *dh_T,
                            void *dx, float *dconv_w, float *dW_a, float *db_a, float *dW_x,
                            float *db_x, float *dLambda, float *dh0, int B, int T, int D, int H,
                            rglru_dtype dt, void *workspace, size_t workspace_bytes,
                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RGLRU_H */
