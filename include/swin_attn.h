/*
 * swin_attn.h - C ABI of the MI355X (gfx950) shifted-window attention library.
 *
 * The library computes one attention module of a Swin Transformer block,
 * W-MSA (no shift) or SW-MSA (shifted windows), forward and backward, over a
 * channels-last latitude-longitude(-level) token grid:
 *
 *   roll the grid by -shift, cut it into windows (row-major window order,
 *   row-major tokens inside a window), project every token to q, k, v,
 *   attend inside each window per head with a relative-position bias and a
 *   shift-region mask, project the head-concatenated output, and put every
 *   token back at its grid position.
 *
 * Sources (titles of the pages this follows):
 *   [TERRA] "TERRA: A Hierarchical Parallel Training and Memory Orchestration
 *           Framework for High-Resolution AI-based Earth Modeling"
 *           - section II-A: fields are B x H x W x C on a regular lat-lon grid;
 *           - section IV-A, Fig. 4: Swin blocks alternate W-MSA and SW-MSA;
 *           - section IV-D: token (u,v) lies in window (u div w, v div w) at
 *             offset (u mod w, v mod w); shifting changes each token's global
 *             coordinate; routes restore tokens at their destination
 *             positions and their backward passes apply the inverse maps;
 *           - section V-A, Eq. 4: windows are flattened in row-major order.
 *   [BEAST] "4D Parallelism Unlocks Exascale Bayesian Neural Networks for
 *           High-Fidelity Atmospheric Modeling"
 *           - "Model Architecture": the domain is rolled by floor(w/2) in both
 *             spatial dimensions between attention layers;
 *           - "Domain-Tensor Parallelism": QKV map, attention per head,
 *             head concatenation;
 *           - mixed precision: bf16 for the attention layers.
 *
 * Readings where the pages are silent (the attention formula itself, scale,
 * bias indexing, roll sign, mask rule, ragged windows) are stated next to the
 * entry points below.
 *
 * Conventions shared by every entry point
 *   - Axis order is (D, H, W) = (level, lat, lon). A 2-D grid has D = 1,
 *     window[0] = 1 and shift[0] = 0.
 *   - Every device pointer is owned by the caller. fwd/bwd never allocate;
 *     only swin_attn_plan_create allocates (its small device tables) and
 *     swin_attn_plan_destroy frees them.
 *   - Calls are asynchronous on the given stream (a hipStream_t; NULL is the
 *     null stream). A plan is immutable after creation and may be used from
 *     several streams at once; concurrent calls must not share workspace.
 *   - Every call validates its arguments before launching anything and
 *     returns a status; nothing aborts or throws across the ABI.
 *     swin_attn_last_error() gives a message for the last failure on the
 *     calling thread.
 */
#ifndef SWIN_ATTN_H_
#define SWIN_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum swin_status {
  SWIN_OK = 0,
  SWIN_ERR_ARG = 1,          /* invalid descriptor, pointer or size */
  SWIN_ERR_UNSUPPORTED = 2,  /* valid, but not implemented for this shape/dtype */
  SWIN_ERR_WORKSPACE = 3,    /* workspace missing or too small */
  SWIN_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} swin_status;

typedef enum swin_dtype {
  SWIN_F32 = 0,   /* fp32 storage and arithmetic (forward only) */
  SWIN_BF16 = 1   /* bf16 storage, fp32 accumulation; fp32 gradients of weights */
} swin_dtype;

/* Periodicity bits (an axis with its bit set wraps around and is not masked). */
#define SWIN_PERIODIC_LEVEL 0x1u
#define SWIN_PERIODIC_LAT   0x2u
#define SWIN_PERIODIC_LON   0x4u

/*
 * Problem descriptor.
 *   ndim      2 (lat, lon) or 3 (level, lat, lon).
 *   dtype     a swin_dtype.
 *   batch     B >= 1. Windows never cross the batch dimension.
 *   grid      (D, H, W), each >= 1; D == 1 when ndim == 2.
 *   channels  C >= 1, C % heads == 0. head_dim = C / heads.
 *   heads     number of attention heads.
 *   window    (wd, wh, ww) with 1 <= w <= grid extent on every axis.
 *   shift     (sd, sh, sw) with 0 <= s < w; all zero is W-MSA. BEAST rolls by
 *             floor(w/2); any s < w is accepted.
 *   periodic  SWIN_PERIODIC_* bits. Longitude wraps around the globe, so the
 *             usual value is SWIN_PERIODIC_LON; latitude and level are then
 *             masked.
 *   scale     logit scale tau; 0 selects head_dim^-1/2.
 */
typedef struct swin_attn_desc {
  int32_t ndim;
  int32_t dtype;
  int64_t batch;
  int64_t grid[3];
  int32_t channels;
  int32_t heads;
  int32_t window[3];
  int32_t shift[3];
  uint32_t periodic;
  float scale;
} swin_attn_desc;

typedef struct swin_attn_plan swin_attn_plan;

/* Host-side statistics of a descriptor's window layout. */
typedef struct swin_attn_stats {
  int64_t n_tokens;       /* B * D * H * W */
  int64_t n_windows;      /* B * prod(ceil(N_a / w_a)) */
  int64_t n_masked;       /* windows whose tokens carry two different wrap labels */
  int64_t n_classes;      /* distinct (extent, label split) window classes */
  int64_t max_tokens;     /* tokens in the largest window */
  int64_t allowed_pairs;  /* (query, key) pairs with equal labels, summed over windows */
} swin_attn_stats;

/*
 * Window layout (host only, needs no GPU).
 *
 * The grid is rolled by -shift: the rolled field is x~[i'] = x[(i'+s) mod N]
 * on every axis (BEAST "Model Architecture" gives the roll by half a window;
 * the sign is this library's reading). Along an axis of extent N, window k
 * covers rolled indices [k*w, min((k+1)*w, N)) for k < ceil(N/w) [TERRA IV-D];
 * the last window of an axis that w does not divide is short and is attended
 * without padding (reading of the ragged edge windows). Windows are numbered
 * row-major over (b, kd, kh, kw) [TERRA V-A, Eq. 4] and tokens inside a
 * window row-major over their local offsets.
 *
 * Wrap labels (reading of the shift-region mask): on a non-periodic axis with
 * s > 0 the last s rolled indices carry label 1, others 0; a query may attend
 * a key only if their labels agree on every axis.
 *
 * swin_attn_host_index_map writes, for every window-major slot t in
 * [0, n_tokens): map[t] = flat grid index (row-major over b, d, h, w) of the
 * token in that slot, and labels[t] = bit a set if the token carries wrap
 * label 1 on axis a. Either output may be NULL. Buffers are host memory of
 * n_tokens elements.
 */
swin_status swin_attn_host_index_map(const swin_attn_desc* desc, int64_t* map, uint8_t* labels);
swin_status swin_attn_host_stats(const swin_attn_desc* desc, swin_attn_stats* out);

/*
 * Plan: validates desc, builds the per-window offset/length table, the window
 * classes and the slot -> grid index map, and uploads them to the current
 * HIP device. Errors: SWIN_ERR_ARG for an invalid descriptor (shift >= window,
 * window > grid, C % heads != 0, ...), SWIN_ERR_UNSUPPORTED for shapes the
 * kernels do not cover (bf16: head_dim 32, 64 or 128, C % 64 == 0, windows of
 * any size, tables of fewer than 2^24 bins per head; fp32: head_dim <= 64 and
 * at most 256 tokens per window), SWIN_ERR_HIP if the upload fails. *out is
 * NULL on error. Windows over 256 tokens, head_dim 64/128 and tables over
 * 2048 bins run on tiled kernels that stream keys and values through LDS with
 * an online softmax [TERRA VII-A: FlashAttention from w >= 32; Table V:
 * head_dim 128].
 */
swin_status swin_attn_plan_create(const swin_attn_desc* desc, swin_attn_plan** out);
void swin_attn_plan_destroy(swin_attn_plan* plan);
swin_status swin_attn_plan_stats(const swin_attn_plan* plan, swin_attn_stats* out);

/*
 * The plan's slot -> grid index map and wrap labels, as swin_attn_host_index_map gives them for
 * the plan's descriptor (same layout and meaning), copied from the plan's host tables: no
 * device call. host_map and host_labels are host buffers of n_tokens elements; either may be
 * NULL. Errors: SWIN_ERR_ARG for a NULL plan.
 */
swin_status swin_attn_index_map(const swin_attn_plan* plan, int64_t* host_map, uint8_t* host_labels);

/*
 * Sizes in bytes of the forward workspace, backward workspace and the saved
 * state that swin_attn_fwd writes for swin_attn_bwd.
 */
swin_status swin_attn_sizes(const swin_attn_plan* plan, size_t* fwd_ws, size_t* bwd_ws, size_t* saved_bytes);

/*
 * Sticky condition flags of a plan: bits that calls on this plan raise on the
 * device and that stay set until cleared, like a floating-point exception flag.
 *   SWIN_FLAG_DT_SATURATED  a backward call's relative-position-bias gradient
 *                           did not fit its fixed-point accumulator (see
 *                           swin_attn_bwd); that call's dbias_table holds NaN.
 * Waits for all work on the plan's device (hipDeviceSynchronize), then writes
 * the flags to *flags (host memory) and, if clear is non-zero, resets them to 0.
 * Not meant for a hot loop; the calls that raise a flag never wait.
 * Errors: SWIN_ERR_ARG for NULL arguments, SWIN_ERR_HIP if the device fails.
 */
#define SWIN_FLAG_DT_SATURATED 0x1u
swin_status swin_attn_plan_flags(const swin_attn_plan* plan, uint32_t* flags, int clear);

/*
 * Forward. Attention reading (the pages name W-MSA/SW-MSA [TERRA IV-A] and
 * give its structure [BEAST "Domain-Tensor Parallelism"] but never its
 * formula): inside each window, for head h,
 *   [q|k|v] = x~ W_qkv^T + b_qkv, head h = columns [h*hd, (h+1)*hd) of each block,
 *   S = tau q_h k_h^T + T[h, bin(i,j)], -inf where labels differ,
 *   o_h = softmax_rows(S) v_h, o = concat_h o_h (head-major channels),
 *   y~ = o W_proj^T + b_proj, and y = y~ put back at the grid positions.
 * bin(i,j) = ((ld_i-ld_j+wd-1)*(2wh-1) + (lh_i-lh_j+wh-1))*(2ww-1) + (lw_i-lw_j+ww-1)
 * over local offsets (query minus key), into a table of (2wd-1)(2wh-1)(2ww-1)
 * entries per head.
 *
 *   x          [B, D, H, W, C] in desc.dtype (device).
 *   w_qkv      [3C, C] (rows: q block, k block, v block; [out, in]).
 *   b_qkv      [3C] or NULL (zero).
 *   w_proj     [C, C] ([out, in]).
 *   b_proj     [C] or NULL.
 *   bias_table fp32 [heads, 2wd-1, 2wh-1, 2ww-1].
 *   y          [B, D, H, W, C] in desc.dtype. Must not alias x.
 *   saved      saved_bytes of device memory for swin_attn_bwd, or NULL for an
 *              inference-only call (then ws must hold at least saved_bytes).
 *   ws         fwd_ws bytes (may be NULL when fwd_ws is 0 and saved is given).
 * Errors: SWIN_ERR_ARG for NULL x/w/y/bias_table, SWIN_ERR_WORKSPACE if ws is
 * too small, SWIN_ERR_HIP if a launch fails.
 */
swin_status swin_attn_fwd(const swin_attn_plan* plan, const void* x, const void* w_qkv, const void* b_qkv,
                          const void* w_proj, const void* b_proj, const float* bias_table, void* y,
                          void* saved, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of swin_attn_fwd, with the same x, weights and bias_table and the
 * saved state it wrote. Gradients are overwritten, never accumulated:
 *   dx           [B, D, H, W, C] in desc.dtype (may alias dy only if ws is separate: it may not).
 *   dw_qkv       fp32 [3C, C];   db_qkv  fp32 [3C] or NULL (not written).
 *   dw_proj      fp32 [C, C];    db_proj fp32 [C] or NULL.
 *   dbias_table  fp32 [heads, 2wd-1, 2wh-1, 2ww-1].
 * dT[h, bin] sums dS over every window and allowed pair (the inverse routes
 * carry gradients back to their sources [TERRA IV-D]); all reductions run in
 * a fixed order (on the tiled kernels every dS term of dT is rounded to an
 * integer multiple of 2^-20 and the integers are summed exactly, in any order),
 * so repeated calls are bitwise identical. On the tiled kernels a dS term of
 * magnitude 2^11 or more (or NaN) does not fit that fixed point: the call then
 * writes NaN over the whole dbias_table and raises SWIN_FLAG_DT_SATURATED in
 * the plan's sticky flags (swin_attn_plan_flags); no status is returned at once,
 * since the call does not wait for its kernels.
 * Tables of more than 8192 bins per head (windows of thousands of tokens) are
 * accumulated with global 64-bit integer atomics instead of workgroup LDS bins:
 * slower, equally exact. Only SWIN_BF16 is supported (SWIN_ERR_UNSUPPORTED for
 * fp32).
 */
swin_status swin_attn_bwd(const swin_attn_plan* plan, const void* dy, const void* x, const void* w_qkv,
                          const void* w_proj, const float* bias_table, const void* saved, void* dx,
                          float* dw_qkv, float* db_qkv, float* dw_proj, float* db_proj, float* dbias_table,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * The module with the smaller saved-state contract: the forward keeps only o and the LSE, and
 * the backward recomputes q, k, v from x with the forward's own QKV GEMM before the usual
 * backward. This trades one QKV product (2 n_tok 3C C FLOPs, not counted as algorithmic) per
 * backward for the q/k/v planes (3 n_tok C elements) that would otherwise stay in device memory
 * from the forward to the backward: activation recomputation, as TERRA section VI's memory
 * orchestration and the Samudra page's activation checkpointing use it to fit deeper models.
 *   swin_attn_sizes_recompute: fwd_ws = the q/k/v planes (the forward's scratch, free after the
 *     call), bwd_ws = the q/k/v planes + swin_attn_sizes' bwd_ws, saved_bytes = o + LSE.
 *   swin_attn_fwd_recompute: as swin_attn_fwd, with saved (saved_bytes, required) holding
 *     [o | LSE] and ws (fwd_ws) the q/k/v planes.
 *   swin_attn_bwd_recompute: as swin_attn_bwd, plus b_qkv (the forward's, NULL for none) to
 *     rebuild q/k/v; saved is the forward's [o | LSE]; ws (bwd_ws) holds the rebuilt planes and
 *     the backward's workspace.
 * Results are bitwise those of swin_attn_fwd / swin_attn_bwd on the same inputs. bf16 only
 * (SWIN_ERR_UNSUPPORTED otherwise); SWIN_ERR_WORKSPACE for a short workspace, SWIN_ERR_ARG for
 * NULL pointers or the aliasing swin_attn_fwd / swin_attn_bwd refuse.
 */
swin_status swin_attn_sizes_recompute(const swin_attn_plan* plan, size_t* fwd_ws, size_t* bwd_ws,
                                      size_t* saved_bytes);
swin_status swin_attn_fwd_recompute(const swin_attn_plan* plan, const void* x, const void* w_qkv, const void* b_qkv,
                                    const void* w_proj, const void* b_proj, const float* bias_table, void* y,
                                    void* saved, void* ws, size_t ws_bytes, void* stream);
swin_status swin_attn_bwd_recompute(const swin_attn_plan* plan, const void* dy, const void* x, const void* w_qkv,
                                    const void* b_qkv, const void* w_proj, const float* bias_table, const void* saved,
                                    void* dx, float* dw_qkv, float* db_qkv, float* dw_proj, float* db_proj,
                                    float* dbias_table, void* ws, size_t ws_bytes, void* stream);

/*
 * swin_attn_bwd without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation). The
 * arguments, results and errors are those of swin_attn_bwd; the workspace is a device array
 * of SWIN_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the process ends.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *   - Plans whose backward workspace (swin_attn_sizes' bwd_ws) exceeds
 *     SWIN_NOALLOC_SCRATCH_BYTES are refused with SWIN_ERR_WORKSPACE; use swin_attn_bwd there.
 *   - The current device must be the plan's device (else SWIN_ERR_ARG).
 *   - Every call on a GPU shares that GPU's scratch array: calls that overlap in time on one
 *     GPU (different streams, or different threads) race on it and must be serialised by the
 *     caller.
 */
#define SWIN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
swin_status swin_attn_bwd_noalloc(const swin_attn_plan* plan, const void* dy, const void* x, const void* w_qkv,
                                  const void* w_proj, const float* bias_table, const void* saved, void* dx,
                                  float* dw_qkv, float* db_qkv, float* dw_proj, float* db_proj, float* dbias_table,
                                  void* stream);

/*
 * Stand-alone cyclic shift + window partition (gather) and its inverse
 * (window reverse + un-shift scatter), on rows of C elements of desc.dtype:
 *   gather:  xw[t, :] = x[map[t], :]     (x on the grid, xw window-major)
 *   scatter: y[map[t], :] = yw[t, :]
 * with map as in swin_attn_host_index_map [TERRA IV-D]. Device pointers,
 * n_tokens * C elements each, no aliasing.
 */
swin_status swin_window_gather(const swin_attn_plan* plan, const void* x, void* xw, void* stream);
swin_status swin_window_scatter(const swin_attn_plan* plan, const void* yw, void* y, void* stream);

/*
 * Stage tracing (a profiling aid for callers that time the library's kernels with HIP
 * events). swin_attn_trace_events installs, for the calling thread, an array of
 * `capacity` hipEvent_t handles (created by the caller) and resets a cursor to 0; from then
 * on every swin_attn_fwd / swin_attn_bwd call on this thread records the next event on its
 * stream at its start and after each of its stages, until the array is full:
 *   forward  (bf16): start | QKV GEMM | attention | proj GEMM                 -> 4 events
 *   backward (bf16): start | weight transposes | dO GEMM | dW_proj GEMM | attention backward
 *                    | dT reduction | dx GEMM | dW_qkv GEMM                   -> 8 events
 * (the recomputing calls record the same; the recomputing backward launches its QKV GEMM before
 * its first event, so that GEMM falls outside the recorded stages)
 * The elapsed time between consecutive events is the duration of that stage. events = NULL
 * uninstalls. swin_attn_trace_cursor returns how many events have been recorded since the
 * last install. Recording failures are reported as SWIN_ERR_HIP by the fwd/bwd call.
 */
swin_status swin_attn_trace_events(void* const* events, int capacity);
int swin_attn_trace_cursor(void);

/* Static message for a status code. */
const char* swin_status_string(swin_status status);
/* Message describing the last failure on the calling thread ("" if none). */
const char* swin_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SWIN_ATTN_H_ */
