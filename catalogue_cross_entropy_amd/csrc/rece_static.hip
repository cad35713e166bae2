// rece_forward_static: the forward pass with its scratch memory in a
// file-scope device array of the library, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).  It enqueues exactly the kernels of rece_forward,
// all on the caller's stream (no second stream or event is created), and
// calls no hipMalloc / hipFree.
//
// The array is per device: each GPU the library runs on holds its own copy
// until the process ends.  Host code never uses the array's name as a device
// address (on the host it is only a stand-in); the address of the current
// device's copy is fetched once per device with hipGetSymbolAddress and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "rece_internal.h"

namespace {

constexpr size_t STATIC_SCRATCH_BYTES = RECE_STATIC_SCRATCH_BYTES;
constexpr int MAX_DEVICES = 64;

static __device__ __align__(256) char scratch[STATIC_SCRATCH_BYTES];

std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};

// Device address of the current device's array (looked up once per device).
rece_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return rece::set_last_error(RECE_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES)
    return rece::set_last_error(RECE_ERR_UNSUPPORTED, "device ordinal beyond the static scratch table");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return rece::set_last_error(RECE_ERR_HIP, e != hipSuccess ? hipGetErrorString(e)
                                                                : "hipGetSymbolAddress returned NULL");
    g_ptr[dev] = ptr;
  }
  *out = g_ptr[dev];
  return RECE_OK;
}

}  // namespace

extern "C" {

rece_status rece_forward_static(rece_plan_t plan, void* stream, const void* X, const void* Y, const int32_t* pos,
                                const void* B, void* saved, float* loss, float* loss_pp) {
  if (!plan) return rece::set_last_error(RECE_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (rece::plan_forward_scratch_bytes(plan) > STATIC_SCRATCH_BYTES)
    return rece::set_last_error(RECE_ERR_WORKSPACE_TOO_SMALL,
                                "the plan's forward scratch exceeds the library's static scratch array (64 MiB)");
  void* ptr = nullptr;
  const rece_status ps = scratch_ptr(&ptr);
  if (ps != RECE_OK) return ps;
  return rece::forward_single_stream(plan, stream, X, Y, pos, B, ptr, saved, loss, loss_pp);
}

}  // extern "C"
