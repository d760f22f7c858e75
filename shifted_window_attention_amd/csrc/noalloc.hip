// The module backward without a caller workspace, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
//
// The workspace that swin_attn_bwd takes from its caller (dO, d(qkv), the transposed weights,
// split-K and bias-gradient partials, the row dot products D) lives here in one file-scope
// device array, `scratch`, of kScratchBytes. Every GPU the library runs on holds its own copy
// until the process ends. Its device address is looked up once per device, with that device
// current, and kept; host code passes that address to the kernels, never the array's name.
// Every call on a GPU reuses that GPU's array: nothing in it needs to start at zero (the
// backward overwrites its partials, and the tiled path clears its fixed-point bias-gradient
// accumulator with a fill kernel), and calls that overlap on one GPU race on it.
#include <mutex>

#include "swin_internal.h"

namespace swin {

constexpr size_t kScratchBytes = SWIN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array (looked up on the first call per device).
static hipError_t scratch_for(int dev, void** out) {
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

using namespace swin;

extern "C" swin_status swin_attn_bwd_noalloc(const swin_attn_plan* plan, const void* dy, const void* x,
                                             const void* w_qkv, const void* w_proj, const float* bias_table,
                                             const void* saved, void* dx, float* dw_qkv, float* db_qkv,
                                             float* dw_proj, float* db_proj, float* dbias_table, void* stream) {
  const swin_status st = bwd_arg_checks(plan, dy, x, w_qkv, w_proj, bias_table, saved, dx, dw_qkv, dw_proj,
                                        dbias_table);
  if (st != SWIN_OK) return st;
  if (plan->bwd_total > kScratchBytes) {
    set_error("backward workspace of " + std::to_string(plan->bwd_total) + " bytes exceeds the " +
              std::to_string(kScratchBytes) + "-byte scratch of swin_attn_bwd_noalloc; use swin_attn_bwd");
    return SWIN_ERR_WORKSPACE;
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error(std::string("hipGetDevice: ") + hipGetErrorString(e));
    return SWIN_ERR_HIP;
  }
  if (dev != plan->device) {
    set_error("the current device is not the plan's device");
    return SWIN_ERR_ARG;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("device index beyond the scratch table");
    return SWIN_ERR_UNSUPPORTED;
  }
  void* ws = nullptr;
  e = scratch_for(dev, &ws);
  if (e == hipSuccess)
    e = launch_bwd_bf16(plan, dy, x, w_qkv, w_proj, bias_table, saved, dx, dw_qkv, db_qkv, dw_proj, db_proj,
                        dbias_table, ws, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_error(std::string("bf16 backward (no allocation): ") + hipGetErrorString(e));
    return SWIN_ERR_HIP;
  }
  return SWIN_OK;
}
