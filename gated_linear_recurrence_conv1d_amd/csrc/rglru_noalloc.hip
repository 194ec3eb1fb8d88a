// rglru_noalloc.hip -- rglru_forward for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same plans and
// kernels as rglru_forward, with the workspace taken from a fixed device array that the library
// owns instead of from the caller.
//
// The array (`scratch`, kNoallocScratchBytes) lives in the code object, so each GPU the library
// runs on holds one copy of it until the process ends. In host code its name is only a stand-in
// for the device symbol, never a device address: the address is looked up once per device with
// hipGetSymbolAddress (on that device's first call, with it current) and only that pointer is
// passed on. Every call on one GPU shares that GPU's array, which keeps the last call's contents;
// the plans clear what must start at zero (look-back words, tickets, the failure count) in their
// own launches, so stale contents never matter. Calls that overlap on one GPU race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "rglru.h"
#include "rglru_launch.h"

namespace {

constexpr size_t kNoallocScratchBytes = size_t{72} << 20;  // 72 MiB
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};  // the array's device address, per device (nullptr: not looked up)

// The current device's copy of the array, looked up on its first use. nullptr on failure.
void *device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

size_t rglru_forward_noalloc_max_bytes(void) { return kNoallocScratchBytes; }

rglru_status rglru_forward_noalloc(const void *x, const void *conv_w, const void *W_a,
                                   const float *b_a, const void *W_x, const float *b_x,
                                   const float *Lambda, const float *h0, void *y, float *h_T,
                                   int B, int T, int D, int H, rglru_dtype dt, void *stream) {
  // the automatic plan's workspace must fit the array (0: invalid shape, rejected below too)
  const size_t need = rglru_forward_workspace_size_planned(B, T, D, H, dt, RGLRU_PLAN_AUTO, 0);
  if (need > kNoallocScratchBytes) return RGLRU_ERR_UNSUPPORTED;
  void *ws = device_scratch();
  if (!ws) return RGLRU_ERR_HIP;
  return rglru_forward_planned(x, conv_w, W_a, b_a, W_x, b_x, Lambda, h0, y, h_T, B, T, D, H, dt,
                               ws, kNoallocScratchBytes, stream, RGLRU_PLAN_AUTO, 0);
}

}  // extern "C"
