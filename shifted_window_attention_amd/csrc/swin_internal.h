// Internal declarations shared by the host plan and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/swin_attn.h"

namespace swin {

// A window class: every window with the same extents and the same wrap-label
// split shares one bias/mask pattern, so a workgroup that handles one class can
// load that pattern once and reuse it for all of its windows.
struct ClassInfo {
  int32_t ext[3];    // window extents along (D, H, W)
  int32_t split[3];  // first local index carrying wrap label 1, or ext[a] if the axis does not split
  int32_t n;         // tokens per window
  int32_t first;     // offset of this class in the class-sorted window list
  int32_t count;     // windows in the class
  int32_t nqt;       // 16-token tiles per window, ceil(n/16)
};

// A contiguous chunk of one class's windows, processed by one workgroup per head. Items of
// the tiled path name one window (first) and one token block of it (count).
struct WorkItem {
  int32_t cls;
  int32_t first;  // offset into the class-sorted window list (tiled path: the window)
  int32_t count;
  int32_t codes;  // tiled path: offset of the class's token-code tables (0 otherwise)
};

// ---- relative-position bins ----
// Linear code of a token's local offsets (ld, lh, lw) in a window with nominal extents
// (wd, wh, ww): code = (ld (2wh-1) + lh) (2ww-1) + lw. The bias-table bin of a query/key pair
// is then code(q) - code(k) + code0 with code0 = code(wd-1, wh-1, ww-1). The wrap-label bits
// (ld >= split_d, lh >= split_h, lw >= split_w) sit above bit 24.
__host__ __device__ inline int token_code(int j, const int* ext, const int* split, const int* win) {
  const int lw = j % ext[2];
  const int r = j / ext[2];
  const int lh = r % ext[1];
  const int ld = r / ext[1];
  const int lab = (ld >= split[0] ? 1 : 0) | (lh >= split[1] ? 2 : 0) | (lw >= split[2] ? 4 : 0);
  return (lab << 24) | ((ld * (2 * win[1] - 1) + lh) * (2 * win[2] - 1) + lw);
}
__host__ __device__ inline int code0_of(const int* win) {
  return ((win[0] - 1) * (2 * win[1] - 1) + (win[1] - 1)) * (2 * win[2] - 1) + (win[2] - 1);
}

// Token codes of the tiled path. Tokens past a window's end take the padding code: a wrap
// label no real token has, so every pair of such a token with a real one is masked (two
// padding tokens share the label, so the kernels also mask on their own validity).
constexpr int kPadCode = 0x7f << 24;
// Relative-position tables of up to kTabLds bins are held in LDS as fp16 in log2 units
// (|error| <= 2^-11 |bias|) with a -inf entry after the last bin, and the codes are then
// staged in an encoding that makes a pair's table address one subtraction and one unsigned
// min:  key side K = 2 local + (label << 16),  query side Q = 2 (local + code0) + (label << 16).
// Q - K is twice the pair's bin when the wrap labels agree and lies outside [0, 2 nbins)
// otherwise; padding tokens take K = kPadK and Q = kPadQ, outside as well, so
// min(Q - K, 2 nbins) (unsigned) addresses the bin's entry or the -inf one. Larger tables are
// read from global memory with the plain codes.
constexpr int kTabLds = 4096;
constexpr int kPadK = 0x40000000, kPadQ = 0x7fffffff;
__host__ __device__ inline int enc_key(int code) { return 2 * (code & 0xffffff) + ((code >> 24) << 16); }
__host__ __device__ inline int enc_query(int code, int code0) {
  return 2 * ((code & 0xffffff) + code0) + ((code >> 24) << 16);
}
// Per class, the plan keeps the key and the query codes of tokens 0 .. kCodeRound-rounded n - 1
// (padding past n), in the encoding above when the table fits LDS, else plain.
constexpr int kCodeRound = 128;

// Work items of one tile count (ceil(n/16)), contiguous in the work list.
struct WorkRange {
  int nqt;
  int begin;
  int count;
};

constexpr int kMaxFwdTiles = 16;  // forward: windows of up to 256 tokens
constexpr int kMaxBwdTiles = 10;  // backward: windows of up to 160 tokens (LDS budget)
constexpr int kFwdMaxChunk = 64;   // windows per forward work item
constexpr int kMaxChunk = 160;     // windows per backward work item
constexpr int kFwdItemOverhead = 2;  // fixed cost of a forward / backward workgroup, in windows
constexpr int kBwdItemOverhead = 4;
constexpr int kMaxBins = 2048;    // bias-table bins per head (windows of <= 256 tokens have < 2048)
constexpr int kTiledMaxBwdBins = 8192;  // tiled backward: bias-gradient bins per head held in LDS (larger
                                        // tables are accumulated with global integer atomics)

struct DevTables {
  int32_t* perm = nullptr;       // [n_tok] window-major slot -> grid row
  int32_t* win_off = nullptr;    // [n_win + 1] token offset of each window (row-major window order)
  int32_t* class_win = nullptr;  // [n_win] window ids sorted by class
  ClassInfo* classes = nullptr;  // [n_cls]
  WorkItem* fwd_work = nullptr;  // [n_fwd_work]
  WorkItem* bwd_work = nullptr;  // [n_bwd_work]
  WorkItem* tiled_work = nullptr;  // [n_tiled_work] (class, window, 64-token block): the tiled dQ kernel
  WorkItem* tiled_kv_work = nullptr;  // (class, window, 128-token block): the tiled forward and dK/dV kernels
  int32_t* tiled_codes = nullptr;     // per class: key codes, then query codes (tiled path)
  unsigned int* flags = nullptr;      // sticky SWIN_FLAG_* bits (swin_attn_plan_flags)
};

}  // namespace swin

struct swin_attn_plan {
  swin_attn_desc d;
  int64_t n_tok = 0, n_win = 0;
  int C = 0, nh = 0, hd = 0;
  int nbins = 0;  // entries per head of the bias table
  float tau = 0.f;
  int device = -1;
  swin_attn_stats stats{};
  std::vector<int32_t> perm, win_off, class_win;
  std::vector<uint8_t> labels;  // slot -> wrap-label bits (host copy, for swin_attn_index_map)
  std::vector<swin::ClassInfo> classes;
  std::vector<swin::WorkItem> fwd_work, bwd_work;
  std::vector<swin::WorkRange> fwd_ranges, bwd_ranges;
  bool tiled = false;                      // bf16 windows over 256 tokens, head_dim 64/128, large tables
  bool tiled_bwd = false;                  // backward on the tiled kernels (tiled, or windows over 160 tokens)
  std::vector<swin::WorkItem> tiled_work, tiled_kv_work;
  std::vector<int32_t> tiled_codes;
  swin::DevTables dev;
  // workspace / saved-state layout (bytes)
  size_t saved_qkv = 0, saved_o = 0, saved_lse = 0, saved_total = 0;
  size_t bwd_do = 0, bwd_dqkv = 0, bwd_wt = 0, bwd_dd = 0, bwd_part = 0, bwd_dbias_part = 0, bwd_total = 0;
  int wgrad_splits_qkv = 1, wgrad_splits_proj = 1;
  int64_t wgrad_chunk_qkv = 0, wgrad_chunk_proj = 0;
};

namespace swin {

void set_error(const std::string& msg);

// Argument checks of the module backward (status and last-error message as the ABI returns them).
swin_status bwd_arg_checks(const swin_attn_plan* plan, const void* dy, const void* x, const void* w_qkv,
                           const void* w_proj, const float* bias_table, const void* saved, const void* dx,
                           const float* dw_qkv, const float* dw_proj, const float* dbias_table);

// Device address of the no-allocation scratch array on device dev (the current device), looked
// up on the first call per device and kept; hipErrorInvalidDevice beyond the per-device table.
hipError_t noalloc_scratch(int dev, void** out);

// Records the next installed trace event (if any) on stream s; see swin_attn_trace_events.
hipError_t trace_mark(hipStream_t s);

// ---- kernel launchers (return hipSuccess or the launch error) ----
hipError_t launch_gather(const swin_attn_plan* p, const void* x, void* xw, bool scatter, hipStream_t s);
hipError_t launch_rows_move(const void* src, void* dst, const int32_t* idx, int64_t n, size_t row_bytes, bool scatter,
                            hipStream_t s);

// bf16 path
hipError_t launch_qkv_fwd_bf16(const swin_attn_plan* p, const void* x, const void* w, const void* b,
                               void* qkv, hipStream_t s);
// Workgroups per CU of the one-tile attention kernels (HIP occupancy query; at least 1).
int attn_fwd_blocks_per_cu(int nqt);
int attn_bwd_blocks_per_cu(int nqt, size_t dyn_lds);
hipError_t launch_attn_fwd_bf16(const swin_attn_plan* p, const void* qkv, const float* table, void* o,
                                float* lse, hipStream_t s);
hipError_t launch_proj_fwd_bf16(const swin_attn_plan* p, const void* o, const void* w, const void* b, void* y,
                                hipStream_t s);
// Module backward; with dx32 set, dx is written there in fp32 instead of to dx (the block's use).
hipError_t launch_bwd_bf16(const swin_attn_plan* p, const void* dy, const void* x, const void* w_qkv,
                           const void* w_proj, const float* table, const void* saved, void* dx, float* dw_qkv,
                           float* db_qkv, float* dw_proj, float* db_proj, float* dtable, void* ws,
                           hipStream_t s, float* dx32 = nullptr);
// launch_bwd_bf16 with the saved q/k/v planes, o rows and LSE given separately (saved is laid out
// [q/k/v | o | LSE]; the recomputing backward rebuilds q/k/v in its workspace instead).
hipError_t launch_bwd_bf16_parts(const swin_attn_plan* p, const void* dy, const void* x, const void* w_qkv,
                                 const void* w_proj, const float* table, const void* qkv, const void* o,
                                 const float* lse, void* dx, float* dw_qkv, float* db_qkv, float* dw_proj,
                                 float* db_proj, float* dtable, void* ws, hipStream_t s, float* dx32 = nullptr);

// Swin block pieces
typedef __bf16 bf16_t;
hipError_t launch_proj_fwd_res_f32(const swin_attn_plan* p, const void* o, const void* w, const void* b,
                                   const void* res, float* h, hipStream_t s);
hipError_t launch_rows_gemm_bf16(const bf16_t* A, int64_t lda, const bf16_t* B, int64_t ldb, int64_t M, int N, int K,
                                 const bf16_t* bias, int mode, bf16_t* out, bf16_t* out2, const bf16_t* aux,
                                 const bf16_t* res, const float* res_f32, float* out_f32, hipStream_t s);
hipError_t launch_wgrad_bf16(const bf16_t* A, int64_t lda, const bf16_t* B, int64_t ldb, int64_t T, int M, int N,
                             int splits, int64_t chunk, float* part, float* dw, float* db, hipStream_t s);
hipError_t launch_transpose_bf16(const void* in, void* out, int R, int Cn, hipStream_t s);
// Layer normalisation of bf16 or fp32 rows (the block's input x, or its fp32 residual stream h).
template <typename TX>
hipError_t launch_layernorm_fwd(const TX* x, const bf16_t* g, const bf16_t* b, bf16_t* y, float* mean, float* rstd,
                                int64_t rows, int C, float eps, hipStream_t s);
// Backward of the layer norm for an fp32 upstream gradient dy plus a residual gradient dres (bf16
// or fp32) over bf16 or fp32 rows x; dx in bf16 and, if dx32 is set, also in fp32.
template <typename TX, typename TR>
hipError_t launch_layernorm_bwd(const float* dy, const TX* x, const float* mean, const float* rstd,
                                const bf16_t* g, const TR* dres, bf16_t* dx, float* dx32, float* part, float* dg,
                                float* db, int64_t rows, int C, hipStream_t s);
// Layer-norm backward partial sums: at most kLnMaxGroups workgroups, each over a contiguous range
// of rows (a multiple of 4, at least 64), so that the final fixed-order reduction stays short.
constexpr int kLnMaxGroups = 1024;
inline int64_t ln_rows_per_group(int64_t rows) {
  int64_t per = (rows + kLnMaxGroups - 1) / kLnMaxGroups;
  per = per < 64 ? 64 : per;
  return (per + 3) / 4 * 4;
}
inline int layernorm_groups(int64_t rows) {
  const int64_t per = ln_rows_per_group(rows);
  return (int)((rows + per - 1) / per);
}
// split-K count and chunk for a token contraction with an M x N output (plan helper)
void wgrad_split(int64_t n_tok, int64_t M, int64_t N, int* splits, int64_t* chunk);

// tiled path (any window size, head_dim 32/64/128)
hipError_t launch_tiled_fwd_bf16(const swin_attn_plan* p, const void* qkv, const float* table, void* o, float* lse,
                                 hipStream_t s);
hipError_t launch_tiled_bwd_bf16(const swin_attn_plan* p, const void* qkv, const float* lse, const void* dO,
                                 const float* dd, const float* table, void* dqkv, unsigned long long* acc,
                                 float* dtable, hipStream_t s);

// fp32 path (forward only)
hipError_t launch_fwd_f32(const swin_attn_plan* p, const void* x, const void* w_qkv, const void* b_qkv,
                          const void* w_proj, const void* b_proj, const float* table, void* y, void* saved,
                          hipStream_t s);

}  // namespace swin
