// Allocation-free forward: loglinear_fwd with its workspace (segment and block
// states, bucket nodes, segment decays) in a file-scope device array instead
// of stream-ordered allocations, for callers that cannot allocate (code under
// HIP graph capture, serving loops, harnesses that forbid hipMalloc).
//
// Each GPU the library runs on holds its own copy of `scratch` from module
// load until the process ends.  On the host the array's name is only a
// stand-in: its device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is handed to the
// kernels.  Every call on one GPU shares the array, so calls that overlap on a
// GPU (different streams, or host threads) race; calls on one stream are
// ordered and safe.  No kernel of the forward expects the workspace to start
// at zero (every element it reads was written earlier in the same call), so
// nothing is cleared.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ll_internal.h"
#include "loglinear.h"

namespace {

static_assert(LOGLINEAR_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must keep 256-byte alignment");

static __device__ __align__(256) unsigned char scratch[LOGLINEAR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (null on a HIP error).
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int loglinear_fwd_noalloc(const void* q, const void* k, const void* v, const float* log_a,
                                     const float* lambda, float* out, int B, int H, int T, int dk,
                                     int dv, int C, void* stream) {
  const ll::ScratchProvider provider{LOGLINEAR_NOALLOC_SCRATCH_BYTES, &scratch_address};
  return ll::fwd_bf16_with_scratch(q, k, v, log_a, lambda, out, B, H, T, dk, dv, C, provider,
                                   static_cast<hipStream_t>(stream));
}
