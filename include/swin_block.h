/*
 * swin_block.h - C ABI of a Swin Transformer block around the shifted-window attention
 * module of swin_attn.h (same library, gfx950, bf16 with fp32 accumulation).
 *
 * [TERRA] section IV-A, Fig. 4: block 0 is W-MSA followed by an MLP, block 1 is SW-MSA
 * followed by an MLP, with layer normalisation in each block. Read as the
 * pre-normalisation Swin block:
 *
 *     h = x + A(LN1(x)),        y = h + W2 GELU(W1 LN2(h) + b1) + b2
 *
 * where A is the attention module of swin_attn.h (its descriptor inside the block
 * descriptor), LN normalises the C channels of a token (biased variance, eps, then a
 * per-channel scale g and shift b) and GELU is the exact a Phi(a). The W-MSA -> SW-MSA pair
 * of the figure is two blocks whose descriptors differ in the shift.
 *
 * Conventions are those of swin_attn.h: caller-owned device memory, asynchronous calls on
 * the given stream, validation before any launch, a status return, no allocation on the
 * forward/backward path (only swin_block_plan_create allocates). Activations are
 * [B, D, H, W, C] bf16; weights bf16 in [out, in] layout; layer-norm scales and shifts bf16
 * [C]; the relative-position table fp32; gradients fp32, overwritten (never accumulated).
 * Inside the block the residual stream h and its gradient are kept in fp32 (only GEMM
 * operands and the outputs y, dx are rounded to bf16), and y = h + W2 (.) + b2 and
 * dx = dh + LN1'(.) are each rounded once.
 */
#ifndef SWIN_BLOCK_H_
#define SWIN_BLOCK_H_

#include "swin_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct swin_block_plan swin_block_plan;

typedef struct swin_block_desc {
  swin_attn_desc attn;  /* the attention module; dtype must be SWIN_BF16, channels <= 1024 */
  int32_t hidden;       /* MLP hidden width; 0 means 4 * channels; a multiple of 64 */
  float ln_eps;         /* layer-norm epsilon; 0 means 1e-5 */
} swin_block_desc;

/* Device pointers of one block's parameters. Biases (b_qkv, b_proj, b1, b2) may be NULL
 * (zero); everything else is required. */
typedef struct swin_block_params {
  const void* ln1_g;   /* [C] */
  const void* ln1_b;   /* [C] */
  const void* w_qkv;   /* [3C, C] */
  const void* b_qkv;   /* [3C] */
  const void* w_proj;  /* [C, C] */
  const void* b_proj;  /* [C] */
  const float* bias_table; /* [heads, 2wd-1, 2wh-1, 2ww-1] fp32 */
  const void* ln2_g;   /* [C] */
  const void* ln2_b;   /* [C] */
  const void* w1;      /* [hidden, C] */
  const void* b1;      /* [hidden] */
  const void* w2;      /* [C, hidden] */
  const void* b2;      /* [C] */
} swin_block_params;

/* fp32 device outputs of the backward, shaped like the parameters; a NULL bias gradient is
 * not written, every other pointer is required. */
typedef struct swin_block_grads {
  float* ln1_g;
  float* ln1_b;
  float* w_qkv;
  float* b_qkv;
  float* w_proj;
  float* b_proj;
  float* bias_table;
  float* ln2_g;
  float* ln2_b;
  float* w1;
  float* b1;
  float* w2;
  float* b2;
} swin_block_grads;

/* Validates the descriptor (everything swin_attn_plan_create checks, plus bf16, C <= 1024 and
 * hidden % 64 == 0) and builds the plan. Errors: SWIN_ERR_ARG, SWIN_ERR_UNSUPPORTED, SWIN_ERR_HIP. */
swin_status swin_block_plan_create(const swin_block_desc* desc, swin_block_plan** out);
void swin_block_plan_destroy(swin_block_plan* plan);

/* Bytes of the forward workspace (0: the forward needs none when saved is given), the backward
 * workspace, and the saved state (what the backward needs: the attention module's saved state,
 * LN1(x), h, LN2(h), the MLP pre-activation and activation, and the layer-norm statistics). */
swin_status swin_block_sizes(const swin_block_plan* plan, size_t* fwd_ws, size_t* bwd_ws, size_t* saved_bytes);

/* The sticky flags of the block's attention module (swin_attn_plan_flags: waits for the device,
 * writes *flags, clears them if clear is non-zero). SWIN_FLAG_DT_SATURATED after a block backward
 * means its bias_table gradient did not fit the fixed-point accumulator and holds NaN. */
swin_status swin_block_plan_flags(const swin_block_plan* plan, uint32_t* flags, int clear);

/* y = block(x). saved receives saved_bytes of state for swin_block_bwd; for an inference call
 * pass saved = NULL and a workspace of at least saved_bytes. y must not alias x.
 * Errors: SWIN_ERR_ARG (NULL plan, params or required pointer; aliasing), SWIN_ERR_WORKSPACE,
 * SWIN_ERR_HIP. */
swin_status swin_block_fwd(const swin_block_plan* plan, const void* x, const swin_block_params* params, void* y,
                           void* saved, void* ws, size_t ws_bytes, void* stream);

/* Backward of swin_block_fwd with the same x and parameters and the saved state it wrote:
 * dx ([B, D, H, W, C] bf16, must not alias dy or x) and every parameter gradient.
 * Reductions run in a fixed order: repeated calls are bitwise identical. Errors as for
 * swin_block_fwd, plus SWIN_ERR_WORKSPACE when ws is smaller than bwd_ws. */
swin_status swin_block_bwd(const swin_block_plan* plan, const void* dy, const void* x,
                           const swin_block_params* params, const void* saved, void* dx,
                           const swin_block_grads* grads, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SWIN_BLOCK_H_ */
