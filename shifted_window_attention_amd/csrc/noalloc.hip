// Scratch memory of the module backward for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid allocation): the entry
// point swin_attn_bwd_noalloc (plan.cpp) runs the backward on it.
//
// The workspace that swin_attn_bwd takes from its caller (dO, d(qkv), the transposed weights,
// split-K and bias-gradient partials, the row dot products D) lives here in one file-scope
// device array, `scratch`, of SWIN_NOALLOC_SCRATCH_BYTES. Every GPU the library runs on holds its
// own copy until the process ends. Its device address is looked up once per device, with that
// device current, and kept; host code passes that address to the kernels, never the array's name.
// Every call on a GPU reuses that GPU's array: nothing in it needs to start at zero (the
// backward overwrites its partials, and the tiled path clears its fixed-point bias-gradient
// accumulator with a fill kernel), and calls that overlap on one GPU race on it.
#include <mutex>

#include "swin_internal.h"

namespace swin {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[SWIN_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

hipError_t noalloc_scratch(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace swin
