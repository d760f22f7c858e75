// Kernel launchers for the host-only sanitizer build (build_host_sanitized.py): each returns
// hipErrorNotSupported without touching its arguments. Linked instead of the HIP sources, they
// let the host code of the library (descriptor checks, window tables, plans without a device,
// route tables, offload argument checks) run under AddressSanitizer and UndefinedBehaviorSanitizer
// on a machine without a GPU. Not part of libswinattn.so.
#include "swin_internal.h"

namespace swin {

hipError_t launch_gather(const swin_attn_plan*, const void*, void*, bool, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_rows_move(const void*, void*, const int32_t*, int64_t, size_t, bool, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_qkv_fwd_bf16(const swin_attn_plan*, const void*, const void*, const void*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_attn_fwd_bf16(const swin_attn_plan*, const void*, const float*, void*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_proj_fwd_bf16(const swin_attn_plan*, const void*, const void*, const void*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_bwd_bf16(const swin_attn_plan*, const void*, const void*, const void*, const void*, const float*,
                           const void*, void*, float*, float*, float*, float*, float*, void*, hipStream_t, float*) {
  return hipErrorNotSupported;
}
hipError_t launch_bwd_bf16_parts(const swin_attn_plan*, const void*, const void*, const void*, const void*,
                                 const float*, const void*, const void*, const float*, void*, float*, float*, float*,
                                 float*, float*, void*, hipStream_t, float*) {
  return hipErrorNotSupported;
}
hipError_t launch_proj_fwd_res_f32(const swin_attn_plan*, const void*, const void*, const void*, const void*, float*,
                                   hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_rows_gemm_bf16(const bf16_t*, int64_t, const bf16_t*, int64_t, int64_t, int, int, const bf16_t*, int,
                                 bf16_t*, bf16_t*, const bf16_t*, const bf16_t*, const float*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_wgrad_bf16(const bf16_t*, int64_t, const bf16_t*, int64_t, int64_t, int, int, int, int64_t, float*,
                             float*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t noalloc_scratch(int, void**) { return hipErrorNotSupported; }
int attn_fwd_blocks_per_cu(int) { return 1; }
int attn_bwd_blocks_per_cu(int, size_t) { return 1; }
hipError_t launch_transpose_bf16(const void*, void*, int, int, hipStream_t) { return hipErrorNotSupported; }
template <typename TX>
hipError_t launch_layernorm_fwd(const TX*, const bf16_t*, const bf16_t*, bf16_t*, float*, float*, int64_t, int, float,
                                hipStream_t) {
  return hipErrorNotSupported;
}
template hipError_t launch_layernorm_fwd<bf16_t>(const bf16_t*, const bf16_t*, const bf16_t*, bf16_t*, float*, float*,
                                                 int64_t, int, float, hipStream_t);
template hipError_t launch_layernorm_fwd<float>(const float*, const bf16_t*, const bf16_t*, bf16_t*, float*, float*,
                                                int64_t, int, float, hipStream_t);
template <typename TX, typename TR>
hipError_t launch_layernorm_bwd(const float*, const TX*, const float*, const float*, const bf16_t*, const TR*, bf16_t*,
                                float*, float*, float*, float*, int64_t, int, hipStream_t) {
  return hipErrorNotSupported;
}
template hipError_t launch_layernorm_bwd<float, bf16_t>(const float*, const float*, const float*, const float*,
                                                        const bf16_t*, const bf16_t*, bf16_t*, float*, float*, float*,
                                                        float*, int64_t, int, hipStream_t);
template hipError_t launch_layernorm_bwd<bf16_t, float>(const float*, const bf16_t*, const float*, const float*,
                                                        const bf16_t*, const float*, bf16_t*, float*, float*, float*,
                                                        float*, int64_t, int, hipStream_t);
hipError_t launch_tiled_fwd_bf16(const swin_attn_plan*, const void*, const float*, void*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_tiled_bwd_bf16(const swin_attn_plan*, const void*, const float*, const void*, const float*,
                                 const float*, void*, unsigned long long*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_fwd_f32(const swin_attn_plan*, const void*, const void*, const void*, const void*, const void*,
                          const float*, void*, void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace swin
