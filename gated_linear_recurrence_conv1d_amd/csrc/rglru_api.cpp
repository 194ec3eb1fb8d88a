// rglru_api.cpp -- the C ABI (include/rglru.h): argument checks, plan choice, workspace layout and
// kernel launches. No allocation, no global state; every call is asynchronous on its stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

#include "rglru.h"
#include "rglru_launch.h"

namespace {

using rglru::kBF16;
using rglru::kF32;

constexpr size_t kAlign = 256;         // workspace carve alignment
// The scan lanes wait on HBM latency, so the chunked plan wants many lanes in flight: chunks of
// about 64 steps (measured best from 1 to 64 sequences of 2560 channels), shorter when that
// still leaves fewer than ~8 waves per SIMD; the direct plan once B * D alone gives 2 waves.
constexpr int kMinChunk = 16;          // smallest chunk the size query provisions for
constexpr int kMaxAutoChunk = 64;      // longest chunk the automatic plan picks
constexpr long long kTargetLanes = 8LL * 64 * 1024;  // ~8 waves per SIMD on 256 CUs x 4 SIMDs
constexpr long long kDirectLanes = 128LL * 1024;     // >= 2 waves per SIMD: scan channels whole

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

size_t elem_bytes(rglru_dtype dt) { return dt == RGLRU_BF16 ? 2 : 4; }

rglru_status check_shape(int B, int T, int D, int H, rglru_dtype dt) {
  if (B < 1 || T < 1 || D < 1 || H < 1) return RGLRU_ERR_INVALID_ARG;
  if (D % H) return RGLRU_ERR_INVALID_ARG;
  if (dt != RGLRU_F32 && dt != RGLRU_BF16) return RGLRU_ERR_UNSUPPORTED;
  if (D / H > 256) return RGLRU_ERR_UNSUPPORTED;
  // element offsets are formed in size_t; grid dims must fit the hardware limits
  if (static_cast<long long>(B) > 65535 || H > 65535) return RGLRU_ERR_UNSUPPORTED;
  return RGLRU_OK;
}

// Chunk length of the chunked plan when the caller leaves it open.
int chunk_for(int B, int T, int D) {
  const long long lanes = static_cast<long long>(B) * D;
  const long long want = (kTargetLanes + lanes - 1) / lanes;
  long long L = (T + want - 1) / want;
  L = std::max<long long>(std::min<long long>(L, kMaxAutoChunk), kMinChunk);
  return L >= T ? T : static_cast<int>(L);
}

// Chunk length of the automatic plan; returns T when the direct plan is chosen.
int auto_chunk(int B, int T, int D) {
  if (static_cast<long long>(B) * D >= kDirectLanes) return T;
  return chunk_for(B, T, D);
}

size_t pre_bytes(int B, int T, int D, rglru_dtype dt) {
  return static_cast<size_t>(B) * T * D * rglru::pre_pair_bytes(dt == RGLRU_BF16 ? kBF16 : kF32);
}

// Scan-stage workspace: chunk summaries [B][nC][D] float2, then carries [B][nC][D] float, then
// the tiled scan's control words (2 + H). The tiled scan (64-step chunks chained by look-back,
// see tiled_scan) puts its look-back words -- one 64-bit word per (tile, channel), B nC D of
// them -- over the summaries.
struct ScanCarve {
  size_t sums, carry, ctrl, total;
};

ScanCarve scan_carve(int B, int D, int H, int nC) {
  ScanCarve c;
  c.sums = 0;
  c.carry = align_up(static_cast<size_t>(B) * nC * D * sizeof(float2));
  c.ctrl = c.carry + align_up(static_cast<size_t>(B) * nC * D * sizeof(float));
  c.total = c.ctrl + rglru::fused_ctrl_bytes(rglru::scan_tiled_groups(D, H));
  return c;
}

// The chunked plan with 64-step chunks on the shapes the fused kernel takes (bf16, Dh in {32,
// 64, 128, 256}) runs as one pass: the fused kernel with the pre-activations read instead of
// computed, its chunks chained by the decoupled look-back. Other chunk lengths and shapes take
// the three passes (summaries, carries, final).
bool tiled_scan(int T, int D, int H, rglru_dtype dt, int L) {
  // the one-pass scan reads each sequence's pre-activations (4 bytes per element) through 32-bit
  // buffer offsets
  return L == 64 && rglru::fused_supported(dt == RGLRU_BF16 ? kBF16 : kF32, T, D, D / H) &&
         static_cast<long long>(T) * D * 4 < (1LL << 32);
}

enum Kind { kDirect, kChunked, kFused };

// Scan-only plan resolution to (direct?, chunk length). Returns false for an invalid request.
bool resolve_plan(int B, int T, int D, rglru_plan plan, int chunk_len, bool &direct, int &L) {
  if (plan == RGLRU_PLAN_AUTO) {
    L = auto_chunk(B, T, D);
    direct = L >= T;
  } else if (plan == RGLRU_PLAN_DIRECT) {
    L = T;
    direct = true;
  } else if (plan == RGLRU_PLAN_CHUNKED) {
    if (chunk_len < 0) return false;
    L = chunk_len == 0 ? chunk_for(B, T, D) : std::min(chunk_len, T);
    direct = false;
  } else {
    return false;
  }
  return true;
}

// Forward plan resolution: FUSED when asked for or (AUTO) when the shape supports it.
rglru_status resolve_forward(int B, int T, int D, int H, rglru_dtype dt, rglru_plan plan,
                             int chunk_len, Kind &kind, int &L) {
  const int io = dt == RGLRU_BF16 ? kBF16 : kF32;
  const bool fusable = rglru::fused_supported(io, T, D, D / H);
  if (plan == RGLRU_PLAN_FUSED || (plan == RGLRU_PLAN_AUTO && fusable)) {
    if (!fusable) return RGLRU_ERR_UNSUPPORTED;
    kind = kFused;
    L = 64;
    return RGLRU_OK;
  }
  bool direct;
  if (!resolve_plan(B, T, D, plan, chunk_len, direct, L)) return RGLRU_ERR_INVALID_ARG;
  kind = direct ? kDirect : kChunked;
  return RGLRU_OK;
}

size_t fused_bytes(int B, int T, int D, int H) {
  return rglru::fused_ctrl_bytes(H) +
         rglru::fused_slots(B, T, H, D / H) * sizeof(unsigned long long);
}

// Workspace of one resolved forward plan. The split plans: control words, pre-activations, then
// (chunked) the scan's chunk summaries; the fused plan: control words, then look-back words.
size_t split_or_fused_bytes(int B, int T, int D, int H, rglru_dtype dt, Kind kind, int L) {
  if (kind == kFused) return align_up(fused_bytes(B, T, D, H));
  return rglru::kCtrlBytes + align_up(pre_bytes(B, T, D, dt)) +
         (kind == kDirect ? 0 : scan_carve(B, D, H, (T + L - 1) / L).total);
}

rglru_status hip_status(hipError_t e) { return e == hipSuccess ? RGLRU_OK : RGLRU_ERR_HIP; }

}  // namespace

extern "C" {

const char *rglru_status_string(rglru_status s) {
  switch (s) {
    case RGLRU_OK: return "ok";
    case RGLRU_ERR_INVALID_ARG: return "invalid argument";
    case RGLRU_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case RGLRU_ERR_WORKSPACE: return "workspace missing or too small";
    case RGLRU_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

size_t rglru_scan_workspace_size(int B, int T, int D, int H, rglru_dtype dt) {
  if (check_shape(B, T, D, H, dt) != RGLRU_OK) return 0;
  return scan_carve(B, D, H, (T + kMinChunk - 1) / kMinChunk).total;
}

size_t rglru_forward_workspace_size(int B, int T, int D, int H, rglru_dtype dt) {
  if (check_shape(B, T, D, H, dt) != RGLRU_OK) return 0;
  const size_t split = rglru::kCtrlBytes + align_up(pre_bytes(B, T, D, dt)) +
                       rglru_scan_workspace_size(B, T, D, H, dt);
  return std::max(split, align_up(fused_bytes(B, T, D, H)));
}

size_t rglru_forward_workspace_size_planned(int B, int T, int D, int H, rglru_dtype dt,
                                            rglru_plan plan, int chunk_len) {
  if (check_shape(B, T, D, H, dt) != RGLRU_OK) return 0;
  Kind kind;
  int L;
  if (resolve_forward(B, T, D, H, dt, plan, chunk_len, kind, L) != RGLRU_OK) return 0;
  return split_or_fused_bytes(B, T, D, H, dt, kind, L);
}

rglru_status rglru_lookback_failures(const void *workspace, size_t workspace_bytes,
                                     unsigned *count, void *stream) {
  if (!workspace || !count || workspace_bytes < rglru::kCtrlBytes) return RGLRU_ERR_INVALID_ARG;
  if (!aligned(workspace, 16)) return RGLRU_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned v = 0;
  (void)hipGetLastError();
  if (hipMemcpyAsync(&v, static_cast<const unsigned *>(workspace) + 1, sizeof(unsigned),
                     hipMemcpyDeviceToHost, s) != hipSuccess)
    return RGLRU_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return RGLRU_ERR_HIP;
  *count = v;
  return RGLRU_OK;
}

rglru_status rglru_forward_plan_info(int B, int T, int D, int H, rglru_dtype dt, int *plan,
                                     int *chunk_len) {
  rglru_status st = check_shape(B, T, D, H, dt);
  if (st != RGLRU_OK) return st;
  if (!plan || !chunk_len) return RGLRU_ERR_INVALID_ARG;
  Kind kind;
  int L;
  st = resolve_forward(B, T, D, H, dt, RGLRU_PLAN_AUTO, 0, kind, L);
  if (st != RGLRU_OK) return st;
  *plan = kind == kFused ? RGLRU_PLAN_FUSED : kind == kDirect ? RGLRU_PLAN_DIRECT : RGLRU_PLAN_CHUNKED;
  *chunk_len = L;
  return RGLRU_OK;
}

}  // extern "C"

namespace {
// rglru_scan_preacts; gave_up (or NULL: a word of the scan's own workspace) counts the look-back
// waits of the tiled scan that gave up.
rglru_status scan_preacts(const void *x, const void *pre, const void *conv_w,
                          const float *Lambda, const float *h0, void *y, float *h_T, int B, int T,
                          int D, int H, rglru_dtype dt, void *workspace, size_t workspace_bytes,
                          void *stream, rglru_plan plan, int chunk_len, unsigned *gave_up) {
  rglru_status st = check_shape(B, T, D, H, dt);
  if (st != RGLRU_OK) return st;
  if (!x || !pre || !conv_w || !Lambda || !y) return RGLRU_ERR_INVALID_ARG;
  const void *vec16[] = {x, pre, conv_w, y};
  for (const void *p : vec16)
    if (!aligned(p, 16)) return RGLRU_ERR_INVALID_ARG;
  const void *vec4[] = {Lambda, h0, h_T};
  for (const void *p : vec4)
    if (p && !aligned(p, 4)) return RGLRU_ERR_INVALID_ARG;
  bool direct;
  int L;
  if (plan == RGLRU_PLAN_FUSED) return RGLRU_ERR_INVALID_ARG;
  if (!resolve_plan(B, T, D, plan, chunk_len, direct, L)) return RGLRU_ERR_INVALID_ARG;
  const size_t io_bytes = static_cast<size_t>(B) * T * D * elem_bytes(dt);
  const size_t pb = pre_bytes(B, T, D, dt);
  if (overlaps(x, io_bytes, y, io_bytes) || overlaps(pre, pb, y, io_bytes))
    return RGLRU_ERR_INVALID_ARG;
  const int nC = direct ? 0 : (T + L - 1) / L;
  if (nC > 65535) return RGLRU_ERR_UNSUPPORTED;  // one grid row per chunk
  const ScanCarve c = scan_carve(B, D, H, nC);
  if (!direct) {
    if (!workspace || workspace_bytes < c.total) return RGLRU_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return RGLRU_ERR_INVALID_ARG;
    if (overlaps(workspace, c.total, y, io_bytes) || overlaps(workspace, c.total, pre, pb) ||
        overlaps(workspace, c.total, x, io_bytes))
      return RGLRU_ERR_INVALID_ARG;
  }
  const int io = dt == RGLRU_BF16 ? kBF16 : kF32;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // start from a clean error state
  if (direct)
    return hip_status(
        rglru::launch_scan_direct(x, pre, conv_w, Lambda, h0, y, h_T, B, T, D, io, s));
  char *ws = static_cast<char *>(workspace);
  if (tiled_scan(T, D, H, dt, L)) {
    unsigned *ctrl = reinterpret_cast<unsigned *>(ws + c.ctrl);
    return hip_status(rglru::launch_scan_tiled(
        x, pre, conv_w, Lambda, h0, y, h_T, B, T, D, H, ctrl, gave_up ? gave_up : ctrl + 1,
        reinterpret_cast<unsigned long long *>(ws + c.sums), s));
  }
  return hip_status(rglru::launch_scan_chunked(x, pre, conv_w, Lambda, h0, y, h_T, B, T, D, L,
                                               reinterpret_cast<float2 *>(ws + c.sums),
                                               reinterpret_cast<float *>(ws + c.carry), io, s));
}
}  // namespace

extern "C" {

rglru_status rglru_scan_preacts(const void *x, const void *pre, const void *conv_w,
                                const float *Lambda, const float *h0, void *y, float *h_T, int B,
                                int T, int D, int H, rglru_dtype dt, void *workspace,
                                size_t workspace_bytes, void *stream, rglru_plan plan,
                                int chunk_len) {
  return scan_preacts(x, pre, conv_w, Lambda, h0, y, h_T, B, T, D, H, dt, workspace,
                      workspace_bytes, stream, plan, chunk_len, nullptr);
}

rglru_status rglru_forward_planned(const void *x, const void *conv_w, const void *W_a,
                                   const float *b_a, const void *W_x, const float *b_x,
                                   const float *Lambda, const float *h0, void *y, float *h_T,
                                   int B, int T, int D, int H, rglru_dtype dt, void *workspace,
                                   size_t workspace_bytes, void *stream, rglru_plan plan,
                                   int chunk_len) {
  rglru_status st = check_shape(B, T, D, H, dt);
  if (st != RGLRU_OK) return st;
  if (!x || !conv_w || !W_a || !b_a || !W_x || !b_x || !Lambda || !y)
    return RGLRU_ERR_INVALID_ARG;
  const void *vec16[] = {x, conv_w, W_a, W_x, y};
  for (const void *p : vec16)
    if (!aligned(p, 16)) return RGLRU_ERR_INVALID_ARG;
  const void *vec4[] = {b_a, b_x, Lambda, h0, h_T};
  for (const void *p : vec4)
    if (p && !aligned(p, 4)) return RGLRU_ERR_INVALID_ARG;
  Kind kind;
  int L;
  st = resolve_forward(B, T, D, H, dt, plan, chunk_len, kind, L);
  if (st != RGLRU_OK) return st;
  const size_t io_bytes = static_cast<size_t>(B) * T * D * elem_bytes(dt);
  if (overlaps(x, io_bytes, y, io_bytes)) return RGLRU_ERR_INVALID_ARG;
  if (kind == kFused) {
    const size_t need = fused_bytes(B, T, D, H);
    if (!workspace || workspace_bytes < need) return RGLRU_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return RGLRU_ERR_INVALID_ARG;
    if (overlaps(workspace, need, y, io_bytes) || overlaps(workspace, need, x, io_bytes))
      return RGLRU_ERR_INVALID_ARG;
    if (static_cast<long long>((T + 63) / 64) * B * H > 0x7fffffffLL) return RGLRU_ERR_UNSUPPORTED;
    (void)hipGetLastError();  // start from a clean error state
    return hip_status(rglru::launch_fused(x, conv_w, W_a, b_a, W_x, b_x, Lambda, h0, y, h_T, B,
                                          T, D, H, workspace, static_cast<hipStream_t>(stream)));
  }
  const bool direct = kind == kDirect;
  const size_t pre_area = rglru::kCtrlBytes + align_up(pre_bytes(B, T, D, dt));
  const size_t need = split_or_fused_bytes(B, T, D, H, dt, kind, L);
  if (!workspace || workspace_bytes < need) return RGLRU_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return RGLRU_ERR_INVALID_ARG;
  if (overlaps(workspace, need, y, io_bytes) || overlaps(workspace, need, x, io_bytes))
    return RGLRU_ERR_INVALID_ARG;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int io = dt == RGLRU_BF16 ? kBF16 : kF32;
  char *ws = static_cast<char *>(workspace);
  char *pre = ws + rglru::kCtrlBytes;
  (void)hipGetLastError();  // start from a clean error state
  // the look-back failure count: zero, bumped only by the tiled scan's waits that give up (its
  // launcher zeroes it; the other scans never wait)
  hipError_t e = hipSuccess;
  if (direct || !tiled_scan(T, D, H, dt, L))
    e = rglru::launch_clear_words(reinterpret_cast<unsigned *>(ws), 2, s);
  if (e == hipSuccess)
    e = rglru::launch_gates(x, conv_w, W_a, b_a, W_x, b_x, pre, B, T, D, H, io, s);
  if (e != hipSuccess) return RGLRU_ERR_HIP;
  return scan_preacts(x, pre, conv_w, Lambda, h0, y, h_T, B, T, D, H, dt, ws + pre_area,
                      workspace_bytes - pre_area, stream,
                      direct ? RGLRU_PLAN_DIRECT : RGLRU_PLAN_CHUNKED, L,
                      reinterpret_cast<unsigned *>(ws) + 1);
}

rglru_status rglru_forward(const void *x, const void *conv_w, const void *W_a, const float *b_a,
                           const void *W_x, const float *b_x, const float *Lambda,
                           const float *h0, void *y, float *h_T, int B, int T, int D, int H,
                           rglru_dtype dt, void *workspace, size_t workspace_bytes,
                           void *stream) {
  return rglru_forward_planned(x, conv_w, W_a, b_a, W_x, b_x, Lambda, h0, y, h_T, B, T, D, H, dt,
                               workspace, workspace_bytes, stream, RGLRU_PLAN_AUTO, 0);
}

rglru_status rglru_gate_preacts(const void *x, const void *conv_w, const void *W_a,
                                const float *b_a, const void *W_x, const float *b_x, void *pre,
                                int B, int T, int D, int H, rglru_dtype dt, void *stream) {
  rglru_status st = check_shape(B, T, D, H, dt);
  if (st != RGLRU_OK) return st;
  if (!x || !conv_w || !W_a || !b_a || !W_x || !b_x || !pre) return RGLRU_ERR_INVALID_ARG;
  const void *vec16[] = {x, conv_w, W_a, W_x, pre};
  for (const void *p : vec16)
    if (!aligned(p, 16)) return RGLRU_ERR_INVALID_ARG;
  const int io = dt == RGLRU_BF16 ? kBF16 : kF32;
  const size_t io_bytes = static_cast<size_t>(B) * T * D * elem_bytes(dt);
  const size_t pre_bytes = static_cast<size_t>(B) * T * D * rglru::pre_pair_bytes(io);
  if (overlaps(x, io_bytes, pre, pre_bytes)) return RGLRU_ERR_INVALID_ARG;
  (void)hipGetLastError();
  return hip_status(rglru::launch_gates(x, conv_w, W_a, b_a, W_x, b_x, pre, B, T, D, H, io,
                                        static_cast<hipStream_t>(stream)));
}

rglru_status rglru_decode_step(const void *x_t, void *conv_state, float *h, void *y_t,
                               const void *conv_w, const void *W_a, const float *b_a,
                               const void *W_x, const float *b_x, const float *Lambda, int N,
                               int D, int H, rglru_dtype dt, void *stream) {
  rglru_status st = check_shape(1, 1, D, H, dt);
  if (st != RGLRU_OK) return st;
  if (N < 1) return RGLRU_ERR_INVALID_ARG;
  if (N > 65535 * 64) return RGLRU_ERR_UNSUPPORTED;
  if (!x_t || !conv_state || !h || !y_t || !conv_w || !W_a || !b_a || !W_x || !b_x || !Lambda)
    return RGLRU_ERR_INVALID_ARG;
  const void *vec16[] = {x_t, conv_state, y_t, conv_w, W_a, W_x};
  for (const void *p : vec16)
    if (!aligned(p, 16)) return RGLRU_ERR_INVALID_ARG;
  const void *vec4[] = {h, b_a, b_x, Lambda};
  for (const void *p : vec4)
    if (!aligned(p, 4)) return RGLRU_ERR_INVALID_ARG;
  const size_t row = static_cast<size_t>(N) * D;
  const size_t eb = elem_bytes(dt);
  if (overlaps(y_t, row * eb, x_t, row * eb) || overlaps(y_t, row * eb, conv_state, 3 * row * eb) ||
      overlaps(y_t, row * eb, h, row * sizeof(float)) ||
      overlaps(conv_state, 3 * row * eb, h, row * sizeof(float)) ||
      overlaps(conv_state, 3 * row * eb, x_t, row * eb) ||
      overlaps(h, row * sizeof(float), x_t, row * eb))
    return RGLRU_ERR_INVALID_ARG;
  const int io = dt == RGLRU_BF16 ? kBF16 : kF32;
  (void)hipGetLastError();
  return hip_status(rglru::launch_decode(x_t, conv_state, h, y_t, conv_w, W_a, b_a, W_x, b_x,
                                         Lambda, N, D, H, io, static_cast<hipStream_t>(stream)));
}

rglru_status rglru_prefill_state(const void *x, void *conv_state, int B, int T, int D,
                                 rglru_dtype dt, void *stream) {
  if (B < 1 || T < 1 || D < 1) return RGLRU_ERR_INVALID_ARG;
  if (dt != RGLRU_F32 && dt != RGLRU_BF16) return RGLRU_ERR_UNSUPPORTED;
  if (!x || !conv_state) return RGLRU_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(conv_state, 16)) return RGLRU_ERR_INVALID_ARG;
  const size_t eb = elem_bytes(dt);
  if (overlaps(x, static_cast<size_t>(B) * T * D * eb, conv_state, static_cast<size_t>(B) * 3 * D * eb))
    return RGLRU_ERR_INVALID_ARG;
  (void)hipGetLastError();
  return hip_status(rglru::launch_prefill_state(x, conv_state, B, T, D,
                                                dt == RGLRU_BF16 ? kBF16 : kF32,
                                                static_cast<hipStream_t>(stream)));
}

rglru_status rglru_local_mqa(const void *q, const void *k, const void *v, void *o, int B, int T,
                             int Hq, int dh, int window, float scale, rglru_dtype dt,
                             void *stream) {
  if (B < 1 || T < 1 || Hq < 1 || dh < 1 || window < 1) return RGLRU_ERR_INVALID_ARG;
  if (dt != RGLRU_BF16 || !rglru::local_mqa_supported(dh)) return RGLRU_ERR_UNSUPPORTED;
  if (B > 65535 || Hq > 65535) return RGLRU_ERR_UNSUPPORTED;
  // one sequence's k (and v) must fit a 32-bit buffer range, with room past it for the kernel's
  // no-op loads
  if (static_cast<size_t>(T) * dh * 2 > (size_t{1} << 30)) return RGLRU_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o) return RGLRU_ERR_INVALID_ARG;
  const void *vec16[] = {q, k, v, o};
  for (const void *p : vec16)
    if (!aligned(p, 16)) return RGLRU_ERR_INVALID_ARG;
  if (!(scale == scale) || scale < 0.0f) return RGLRU_ERR_INVALID_ARG;  // NaN or negative
  const size_t qbytes = static_cast<size_t>(B) * T * Hq * dh * 2;
  const size_t kbytes = static_cast<size_t>(B) * T * dh * 2;
  if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kbytes) || overlaps(o, qbytes, v, kbytes))
    return RGLRU_ERR_INVALID_ARG;
  if (scale == 0.0f) scale = 1.0f / std::sqrt(static_cast<float>(dh));
  (void)hipGetLastError();
  return hip_status(rglru::launch_local_mqa(q, k, v, o, B, T, Hq, dh, window, scale,
                                            static_cast<hipStream_t>(stream)));
}

size_t rglru_backward_workspace_size(int B, int T, int D, int H, rglru_dtype dt) {
  if (check_shape(B, T, D, H, dt) != RGLRU_OK) return 0;
  return rglru::backward_layout(B, T, D, H, dt == RGLRU_BF16 ? kBF16 : kF32).total;
}

rglru_status rglru_backward(const void *x, const void *conv_w, const void *W_a, const float *b_a,
                            const void *W_x, const float *b_x, const float *Lambda,
                            const float *h0, const void *y, const void *dy, const float *dh_T,
                            void *dx, float *dconv_w, float *dW_a, float *db_a, float *dW_x,
                            float *db_x, float *dLambda, float *dh0, int B, int T, int D, int H,
                            rglru_dtype dt, void *workspace, size_t workspace_bytes,
                            void *stream) {
  rglru_status st = check_shape(B, T, D, H, dt);
  if (st != RGLRU_OK) return st;
  if (!x || !conv_w || !W_a || !b_a || !W_x || !b_x || !Lambda || !y || !dy || !dx ||
      !dconv_w || !dW_a || !db_a || !dW_x || !db_x || !dLambda)
    return RGLRU_ERR_INVALID_ARG;
  const void *vec16[] = {x, conv_w, W_a, W_x, y, dy, dx};
  for (const void *p : vec16)
    if (!aligned(p, 16)) return RGLRU_ERR_INVALID_ARG;
  const void *vec4[] = {b_a, b_x, Lambda, h0, dh_T, dconv_w, dW_a, db_a, dW_x, db_x, dLambda, dh0};
  for (const void *p : vec4)
    if (p && !aligned(p, 4)) return RGLRU_ERR_INVALID_ARG;
  const int io = dt == RGLRU_BF16 ? kBF16 : kF32;
  const rglru::BwdLayout L = rglru::backward_layout(B, T, D, H, io);
  if (L.nC > 65535) return RGLRU_ERR_UNSUPPORTED;  // one grid row per chunk
  if (static_cast<long long>(B) * T >= (1LL << 31)) return RGLRU_ERR_UNSUPPORTED;  // row index
  if (!workspace || workspace_bytes < L.total) return RGLRU_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return RGLRU_ERR_INVALID_ARG;
  // outputs must not overlap the inputs, the workspace or each other
  const size_t io_bytes = static_cast<size_t>(B) * T * D * elem_bytes(dt);
  const size_t wbytes = static_cast<size_t>(H) * (D / H) * (D / H) * sizeof(float);
  const size_t dvec = static_cast<size_t>(D) * sizeof(float);
  const size_t bd = static_cast<size_t>(B) * D * sizeof(float);
  struct Span {
    const void *p;
    size_t n;
  };
  const Span outs[] = {{dx, io_bytes}, {dconv_w, 4 * dvec}, {dW_a, wbytes}, {db_a, dvec},
                       {dW_x, wbytes}, {db_x, dvec},        {dLambda, dvec}, {dh0, bd}};
  const size_t pbytes = static_cast<size_t>(D / H) * (D / H) * elem_bytes(dt) * H;
  const Span ins[] = {{x, io_bytes},  {y, io_bytes},   {dy, io_bytes},   {conv_w, 4 * D * elem_bytes(dt)},
                      {W_a, pbytes},  {W_x, pbytes},   {b_a, dvec},      {b_x, dvec},
                      {Lambda, dvec}, {h0, bd},        {dh_T, bd},       {workspace, L.total}};
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
    for (size_t j = 0; j < sizeof(ins) / sizeof(ins[0]); ++j)
      if (overlaps(outs[i].p, outs[i].n, ins[j].p, ins[j].n)) return RGLRU_ERR_INVALID_ARG;
    for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
      if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return RGLRU_ERR_INVALID_ARG;
  }
  (void)hipGetLastError();
  return hip_status(rglru::launch_backward(x, conv_w, W_a, b_a, W_x, b_x, Lambda, h0, y, dy, dh_T,
                                           dx, dconv_w, dW_a, db_a, dW_x, db_x, dLambda, dh0, B,
                                           T, D, H, io, workspace,
                                           static_cast<hipStream_t>(stream)));
}

}  // extern "C"
