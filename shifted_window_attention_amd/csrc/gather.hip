// Stand-alone cyclic shift + window partition (gather) and window reverse + un-shift
// (scatter). Rows are moved whole: a window-major slot t takes grid row perm[t]
// (TERRA section IV-D: a token's global coordinate fixes its window and offset;
// the reverse route restores every token at its position).
//
// HBM-bound: each launch reads and writes N_tok * C * elem bytes once. One
// workgroup moves 16 rows; every lane copies 16-byte chunks, so each row is read
// and written as contiguous, fully coalesced segments.
#include "device_common.h"
#include "swin_internal.h"

namespace swin {

template <bool kScatter>
__global__ __launch_bounds__(256) void k_window_move(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                     const int32_t* __restrict__ perm, int64_t n_tok,
                                                     int chunks_per_row) {
  const int rows_per_block = 16;
  const int64_t row0 = (int64_t)blockIdx.x * rows_per_block;
  const int total = rows_per_block * chunks_per_row;
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    const int r = i / chunks_per_row;
    const int c = i - r * chunks_per_row;
    const int64_t t = row0 + r;
    if (t >= n_tok) break;
    const int64_t g = perm[t];
    if (kScatter)
      dst[g * chunks_per_row + c] = src[t * chunks_per_row + c];
    else
      dst[t * chunks_per_row + c] = src[g * chunks_per_row + c];
  }
}

template <bool kScatter>
__global__ __launch_bounds__(256) void k_window_move_u16(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                         const int32_t* __restrict__ perm, int64_t n_tok, int row) {
  const int64_t t = blockIdx.x;
  if (t >= n_tok) return;
  const int64_t g = perm[t];
  for (int c = threadIdx.x; c < row; c += blockDim.x) {
    if (kScatter)
      dst[g * row + c] = src[t * row + c];
    else
      dst[t * row + c] = src[g * row + c];
  }
}

// Rows of row_bytes bytes: dst[i] = src[idx[i]] (gather) or dst[idx[i]] = src[i] (scatter),
// i < n. 16-byte chunks when rows and pointers allow it, 2-byte words otherwise.
hipError_t launch_rows_move(const void* src, void* dst, const int32_t* idx, int64_t n, size_t row_bytes, bool scatter,
                            hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (row_bytes % 16 == 0 && ((uintptr_t)src % 16) == 0 && ((uintptr_t)dst % 16) == 0) {
    const int chunks = (int)(row_bytes / 16);
    const unsigned blocks = (unsigned)((n + 15) / 16);
    if (scatter)
      k_window_move<true><<<blocks, 256, 0, s>>>((const uint4*)src, (uint4*)dst, idx, n, chunks);
    else
      k_window_move<false><<<blocks, 256, 0, s>>>((const uint4*)src, (uint4*)dst, idx, n, chunks);
  } else {
    const int row = (int)(row_bytes / 2);
    if (scatter)
      k_window_move_u16<true><<<(unsigned)n, 64, 0, s>>>((const uint16_t*)src, (uint16_t*)dst, idx, n, row);
    else
      k_window_move_u16<false><<<(unsigned)n, 64, 0, s>>>((const uint16_t*)src, (uint16_t*)dst, idx, n, row);
  }
  return hipGetLastError();
}

hipError_t launch_gather(const swin_attn_plan* p, const void* x, void* xw, bool scatter, hipStream_t s) {
  const size_t es = p->d.dtype == SWIN_BF16 ? 2 : 4;
  return launch_rows_move(x, xw, p->dev.perm, p->n_tok, (size_t)p->C * es, scatter, s);
}

}  // namespace swin
