// Host side of the Swin block (include/swin_block.h): plan, workspace layout and the launch
// sequences of the forward and backward passes.
#include <algorithm>
#include <new>
#include <string>

#include "../../include/swin_block.h"
#include "swin_internal.h"

using swin::bf16_t;

struct swin_block_plan {
  swin_attn_plan* attn = nullptr;
  int C = 0, H = 0;
  float eps = 1e-5f;
  int64_t T = 0;
  // saved state (byte offsets)
  size_t s_xn1 = 0, s_h = 0, s_xn2 = 0, s_a1 = 0, s_g1 = 0, s_st1 = 0, s_st2 = 0, s_total = 0;
  // backward workspace (byte offsets; the attention module's workspace comes first)
  size_t w_dh = 0, w_dh32 = 0, w_dxn32 = 0, w_da1 = 0, w_w1t = 0, w_w2t = 0, w_ln = 0, w_part = 0, w_total = 0;
  int split_w1 = 1, split_w2 = 1;
  int64_t chunk_w1 = 0, chunk_w2 = 0;
};

namespace {

swin_status fail(swin_status st, const std::string& msg) {
  swin::set_error(msg);
  return st;
}

swin_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SWIN_OK;
  swin::set_error(std::string(what) + ": " + hipGetErrorString(e));
  return SWIN_ERR_HIP;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

extern "C" {

swin_status swin_block_plan_create(const swin_block_desc* desc, swin_block_plan** out) {
  if (!out) return fail(SWIN_ERR_ARG, "plan output is NULL");
  *out = nullptr;
  if (!desc) return fail(SWIN_ERR_ARG, "descriptor is NULL");
  if (desc->attn.dtype != SWIN_BF16) return fail(SWIN_ERR_UNSUPPORTED, "the block is implemented for bf16 only");
  if (desc->attn.channels > 1024) return fail(SWIN_ERR_UNSUPPORTED, "the block supports channels <= 1024");
  const int H = desc->hidden > 0 ? desc->hidden : 4 * desc->attn.channels;
  if (desc->hidden < 0 || H % 64 != 0) return fail(SWIN_ERR_UNSUPPORTED, "hidden width must be a multiple of 64");
  if (!(desc->ln_eps >= 0.f)) return fail(SWIN_ERR_ARG, "ln_eps must be >= 0");
  swin_attn_plan* ap = nullptr;
  swin_status st = swin_attn_plan_create(&desc->attn, &ap);
  if (st != SWIN_OK) return st;
  swin_block_plan* p = new (std::nothrow) swin_block_plan();
  if (!p) {
    swin_attn_plan_destroy(ap);
    return fail(SWIN_ERR_ARG, "out of host memory");
  }
  p->attn = ap;
  p->C = desc->attn.channels;
  p->H = H;
  p->eps = desc->ln_eps > 0.f ? desc->ln_eps : 1e-5f;
  const int64_t T = ap->n_tok;
  p->T = T;
  // the residual stream h and its gradient stay in fp32 (act32); GEMM operands are bf16 (act)
  const size_t act = align256((size_t)T * p->C * 2), act32 = align256((size_t)T * p->C * 4),
               hid = align256((size_t)T * H * 2), sts = align256((size_t)T * 8);
  size_t o = align256(ap->saved_total);
  p->s_xn1 = o; o += act;
  p->s_h = o; o += act32;
  p->s_xn2 = o; o += act;
  p->s_a1 = o; o += hid;
  p->s_g1 = o; o += hid;
  p->s_st1 = o; o += sts;
  p->s_st2 = o; o += sts;
  p->s_total = o;
  swin::wgrad_split(T, H, p->C, &p->split_w1, &p->chunk_w1);
  swin::wgrad_split(T, p->C, H, &p->split_w2, &p->chunk_w2);
  o = align256(ap->bwd_total);
  p->w_dh = o; o += act;
  p->w_dh32 = o; o += act32;
  p->w_dxn32 = o; o += act32;
  p->w_da1 = o; o += hid;
  p->w_w1t = o; o += align256((size_t)H * p->C * 2);
  p->w_w2t = o; o += align256((size_t)H * p->C * 2);
  p->w_ln = o; o += align256((size_t)swin::layernorm_groups(T) * 2 * p->C * 4);
  p->w_part = o;
  o += align256(std::max((size_t)p->split_w1 * ((size_t)H * p->C + H), (size_t)p->split_w2 * ((size_t)H * p->C + p->C)) * 4);
  p->w_total = o;
  *out = p;
  return SWIN_OK;
}

void swin_block_plan_destroy(swin_block_plan* plan) {
  if (!plan) return;
  swin_attn_plan_destroy(plan->attn);
  delete plan;
}

swin_status swin_block_plan_flags(const swin_block_plan* plan, uint32_t* flags, int clear) {
  if (!plan) return fail(SWIN_ERR_ARG, "plan is NULL");
  return swin_attn_plan_flags(plan->attn, flags, clear);
}

swin_status swin_block_sizes(const swin_block_plan* plan, size_t* fwd_ws, size_t* bwd_ws, size_t* saved_bytes) {
  if (!plan) return fail(SWIN_ERR_ARG, "plan is NULL");
  if (fwd_ws) *fwd_ws = 0;
  if (bwd_ws) *bwd_ws = plan->w_total;
  if (saved_bytes) *saved_bytes = plan->s_total;
  return SWIN_OK;
}

swin_status swin_block_fwd(const swin_block_plan* plan, const void* x, const swin_block_params* prm, void* y,
                           void* saved, void* ws, size_t ws_bytes, void* stream) {
  if (!plan || !prm) return fail(SWIN_ERR_ARG, "NULL plan or parameters");
  if (!x || !y || !prm->ln1_g || !prm->ln1_b || !prm->w_qkv || !prm->w_proj || !prm->bias_table || !prm->ln2_g ||
      !prm->ln2_b || !prm->w1 || !prm->w2)
    return fail(SWIN_ERR_ARG, "NULL input, output or parameter pointer");
  if (x == y) return fail(SWIN_ERR_ARG, "y must not alias x");
  char* sv = (char*)saved;
  if (!sv) {
    if (!ws || ws_bytes < plan->s_total) return fail(SWIN_ERR_WORKSPACE, "inference call needs a workspace of saved_bytes");
    sv = (char*)ws;
  }
  const swin_attn_plan* ap = plan->attn;
  hipStream_t s = (hipStream_t)stream;
  const int C = plan->C, H = plan->H;
  const int64_t T = plan->T;
  bf16_t* xn1 = (bf16_t*)(sv + plan->s_xn1);
  float* h = (float*)(sv + plan->s_h);
  bf16_t* xn2 = (bf16_t*)(sv + plan->s_xn2);
  bf16_t* a1 = (bf16_t*)(sv + plan->s_a1);
  bf16_t* g1 = (bf16_t*)(sv + plan->s_g1);
  float* st1 = (float*)(sv + plan->s_st1);
  float* st2 = (float*)(sv + plan->s_st2);
  // the attention module's saved state (q/k/v planes, o, lse) leads the block's
  void* qkv = sv;
  void* o = sv + ap->saved_qkv;
  float* lse = (float*)(sv + ap->saved_qkv + ap->saved_o);

  hipError_t e = swin::launch_layernorm_fwd<bf16_t>((const bf16_t*)x, (const bf16_t*)prm->ln1_g,
                                                    (const bf16_t*)prm->ln1_b, xn1, st1, st1 + T, T, C, plan->eps, s);
  if (e == hipSuccess) e = swin::launch_qkv_fwd_bf16(ap, xn1, prm->w_qkv, prm->b_qkv, qkv, s);
  if (e == hipSuccess) e = swin::launch_attn_fwd_bf16(ap, qkv, prm->bias_table, o, lse, s);
  // h = x + proj(o), kept in fp32
  if (e == hipSuccess) e = swin::launch_proj_fwd_res_f32(ap, o, prm->w_proj, prm->b_proj, x, h, s);
  if (e == hipSuccess)
    e = swin::launch_layernorm_fwd<float>(h, (const bf16_t*)prm->ln2_g, (const bf16_t*)prm->ln2_b, xn2, st2, st2 + T,
                                          T, C, plan->eps, s);
  if (e == hipSuccess)
    e = swin::launch_rows_gemm_bf16(xn2, C, (const bf16_t*)prm->w1, C, T, H, C, (const bf16_t*)prm->b1, 2, g1, a1,
                                    nullptr, nullptr, nullptr, nullptr, s);
  // y = h + W2 g1 + b2, one rounding
  if (e == hipSuccess)
    e = swin::launch_rows_gemm_bf16(g1, H, (const bf16_t*)prm->w2, H, T, C, H, (const bf16_t*)prm->b2, 0, (bf16_t*)y,
                                    nullptr, nullptr, nullptr, h, nullptr, s);
  return hip_status(e, "block forward");
}

swin_status swin_block_bwd(const swin_block_plan* plan, const void* dy, const void* x,
                           const swin_block_params* prm, const void* saved, void* dx,
                           const swin_block_grads* gr, void* ws, size_t ws_bytes, void* stream) {
  if (!plan || !prm || !gr) return fail(SWIN_ERR_ARG, "NULL plan, parameters or gradients");
  if (!dy || !x || !saved || !dx || !prm->ln1_g || !prm->ln1_b || !prm->w_qkv || !prm->w_proj || !prm->bias_table ||
      !prm->ln2_g || !prm->ln2_b || !prm->w1 || !prm->w2)
    return fail(SWIN_ERR_ARG, "NULL input, output or parameter pointer");
  if (!gr->ln1_g || !gr->ln1_b || !gr->w_qkv || !gr->w_proj || !gr->bias_table || !gr->ln2_g || !gr->ln2_b ||
      !gr->w1 || !gr->w2)
    return fail(SWIN_ERR_ARG, "NULL gradient pointer");
  if (dx == dy || dx == x) return fail(SWIN_ERR_ARG, "dx must not alias dy or x");
  if (!ws || ws_bytes < plan->w_total) return fail(SWIN_ERR_WORKSPACE, "backward workspace too small");
  const swin_attn_plan* ap = plan->attn;
  hipStream_t s = (hipStream_t)stream;
  const int C = plan->C, H = plan->H;
  const int64_t T = plan->T;
  const char* sv = (const char*)saved;
  const bf16_t* xn1 = (const bf16_t*)(sv + plan->s_xn1);
  const float* h = (const float*)(sv + plan->s_h);
  const bf16_t* xn2 = (const bf16_t*)(sv + plan->s_xn2);
  const bf16_t* a1 = (const bf16_t*)(sv + plan->s_a1);
  const bf16_t* g1 = (const bf16_t*)(sv + plan->s_g1);
  const float* st1 = (const float*)(sv + plan->s_st1);
  const float* st2 = (const float*)(sv + plan->s_st2);
  char* w = (char*)ws;
  bf16_t* dh = (bf16_t*)(w + plan->w_dh);
  float* dh32 = (float*)(w + plan->w_dh32);
  float* dxn = (float*)(w + plan->w_dxn32);  // dLN2-out, then dLN1-out, in fp32
  bf16_t* da1 = (bf16_t*)(w + plan->w_da1);
  bf16_t* w1t = (bf16_t*)(w + plan->w_w1t);
  bf16_t* w2t = (bf16_t*)(w + plan->w_w2t);
  float* lnpart = (float*)(w + plan->w_ln);
  float* part = (float*)(w + plan->w_part);

  // MLP: da1 = (dy W2) * GELU'(a1); dW2 = dy^T g1, db2 = sum dy; dW1 = da1^T xn2, db1 = sum da1;
  // dxn2 = da1 W1
  hipError_t e = swin::launch_transpose_bf16(prm->w1, w1t, H, C, s);
  if (e == hipSuccess) e = swin::launch_transpose_bf16(prm->w2, w2t, C, H, s);
  if (e == hipSuccess)
    e = swin::launch_rows_gemm_bf16((const bf16_t*)dy, C, w2t, C, T, H, C, nullptr, 3, da1, nullptr, a1, nullptr,
                                    nullptr, nullptr, s);
  if (e == hipSuccess)
    e = swin::launch_wgrad_bf16((const bf16_t*)dy, C, g1, H, T, C, H, plan->split_w2, plan->chunk_w2, part, gr->w2,
                                gr->b2, s);
  if (e == hipSuccess)
    e = swin::launch_wgrad_bf16(da1, H, xn2, C, T, H, C, plan->split_w1, plan->chunk_w1, part, gr->w1, gr->b1, s);
  if (e == hipSuccess)
    e = swin::launch_rows_gemm_bf16(da1, H, w1t, H, T, C, H, nullptr, 0, nullptr, nullptr, nullptr, nullptr, nullptr,
                                    dxn, s);
  // LN2: dh = dy + LN2'(dxn2), in bf16 for the attention module's products and in fp32 for
  // the residual add of LN1's backward
  if (e == hipSuccess)
    e = swin::launch_layernorm_bwd<float, bf16_t>(dxn, h, st2, st2 + T, (const bf16_t*)prm->ln2_g, (const bf16_t*)dy,
                                                  dh, dh32, lnpart, gr->ln2_g, gr->ln2_b, T, C, s);
  if (e != hipSuccess) return hip_status(e, "block backward (MLP)");
  // attention module with dy = dh on its input LN1(x); dxn1 reuses the dxn buffer
  e = swin::launch_bwd_bf16(ap, dh, xn1, prm->w_qkv, prm->w_proj, prm->bias_table, sv, nullptr, gr->w_qkv,
                            gr->b_qkv, gr->w_proj, gr->b_proj, gr->bias_table, w, s, dxn);
  // LN1: dx = dh + LN1'(dxn1), one rounding
  if (e == hipSuccess)
    e = swin::launch_layernorm_bwd<bf16_t, float>(dxn, (const bf16_t*)x, st1, st1 + T, (const bf16_t*)prm->ln1_g, dh32,
                                                  (bf16_t*)dx, nullptr, lnpart, gr->ln1_g, gr->ln1_b, T, C, s);
  return hip_status(e, "block backward");
}

}  // extern "C"
