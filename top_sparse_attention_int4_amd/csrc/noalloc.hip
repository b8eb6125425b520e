// twl_decode_noalloc: the decode step with its workspace in a static device array, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on holds its own copy from
// module load until the process ends.  In host code the name is only a host-side stand-in, never a
// device address, so its device address is looked up once per device (hipGetSymbolAddress, with that
// device current, on the entry point's first call there) and that address is what the kernels get.
// The decode's kernels initialise every workspace word they read, so nothing is cleared here; calls
// that overlap on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "twl.h"
#include "twl_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)TWL_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of this device's `scratch`, looked up on the first call per device.
twl_status scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TWL_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return TWL_EUNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TWL_EHIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return TWL_OK;
}

}  // namespace

extern "C" twl_status twl_decode_noalloc(const twl_cache* cache, const void* q, const twl_decode_params* params,
                                         float* out, float* lse, float* threshold, int32_t* sel_indptr,
                                         int32_t* sel_tokens, int64_t capacity, void* stream) {
  size_t need = 0;
  twl_status st = twl::decode_workspace_need(cache, q, params, out, sel_indptr, sel_tokens, capacity, &need);
  if (st != TWL_OK) return st;
  if (need > kScratchBytes) return TWL_EWORKSPACE;
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != TWL_OK) return st;
  return twl::decode_with_workspace(cache, q, params, out, lse, threshold, sel_indptr, sel_tokens, capacity, ws,
                                    kScratchBytes, stream);
}
