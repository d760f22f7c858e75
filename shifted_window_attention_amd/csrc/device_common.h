// Device helpers for gfx950 (CDNA4): bf16 vectors, MFMA wrappers, conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swin {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// D(16x16) += A(16x32) B(32x16). Lane l holds A row l%16, B column l%16, each with 8
// consecutive k values of group l/16; D column l%16, rows 4*(l/16) + r.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// D(32x32) += A(32x16) B(16x32). Lane l holds A row l%32 / B column l%32 with k group l/32;
// D column l%32, rows 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp32 -> bf16 round-to-nearest-even (hardware conversion on gfx950).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float wave_max_xor16_32(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float wave_sum_xor16_32(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// ---- relative-position bins ----
// Linear code of a token's local offsets (ld, lh, lw) in a window with nominal extents
// (wd, wh, ww): code = (ld (2wh-1) + lh) (2ww-1) + lw. The bias-table bin of a query/key pair
// is then code(q) - code(k) + code0 with code0 = code(wd-1, wh-1, ww-1). The wrap-label bits
// (ld >= split_d, lh >= split_h, lw >= split_w) sit above bit 24.
__device__ __forceinline__ int token_code(int j, const int* ext, const int* split, const int* win) {
  const int lw = j % ext[2];
  const int r = j / ext[2];
  const int lh = r % ext[1];
  const int ld = r / ext[1];
  const int lab = (ld >= split[0] ? 1 : 0) | (lh >= split[1] ? 2 : 0) | (lw >= split[2] ? 4 : 0);
  return (lab << 24) | ((ld * (2 * win[1] - 1) + lh) * (2 * win[2] - 1) + lw);
}
__device__ __forceinline__ int code0_of(const int* win) {
  return ((win[0] - 1) * (2 * win[1] - 1) + (win[1] - 1)) * (2 * win[2] - 1) + (win[2] - 1);
}
// Logit offset (log2 units) of a pair from the two tokens' codes: -inf across wrap labels.
__device__ __forceinline__ float pair_bias_codes(int cq, int ck, int code0, const float* tab2) {
  if ((cq >> 24) != (ck >> 24)) return -INFINITY;
  return tab2[(cq & 0xffffff) - (ck & 0xffffff) + code0];
}

// ---- LDS tiles of 32-element bf16 head rows (64 bytes per row) ----
// A tile row holds four 16-byte chunks; physical slot s of row r holds logical chunk
// s ^ swz(r). With this swizzle the 16-byte fragment reads of 8 or 16 consecutive rows at
// one logical chunk touch distinct banks.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// Byte offset of element `col` (multiple of 4) of row r in a swizzled tile.
__device__ __forceinline__ int swz_off(int r, int col) {
  return r * 64 + 16 * ((col >> 3) ^ swz(r)) + 2 * (col & 7);
}

// 16-byte fragment (logical chunk c, i.e. columns 8c..8c+7) of row r.
__device__ __forceinline__ bf16x8 tile_frag(const unsigned char* tile, int r, int c) {
  return *(const bf16x8*)(tile + r * 64 + 16 * (c ^ swz(r)));
}

// Four bf16 through gfx950's transposing LDS read: lane i of each 16-lane group receives
// element (i % 4) of the 8-byte pieces addressed by lanes 4r + i/4, r = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr(const void* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// MFMA 16x16x32 operand with 8 k values for column col0 + li of a swizzled tile whose rows
// are k: rows row0 + 4g + r (r < 4) and row0 + 16 + 4g + r.
__device__ __forceinline__ bf16x8 tile_frag_tr(const unsigned char* tile, int row0, int col0, int g, int li) {
  const int r = row0 + 4 * g + (li >> 2);
  const int col = col0 + 4 * (li & 3);
  const bf16x4 lo = lds_read_tr(tile + swz_off(r, col));
  const bf16x4 hi = lds_read_tr(tile + swz_off(r + 16, col));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Buffer resource over `bytes` bytes at `base` (raw buffer, 32-bit elements format as the
// CDNA buffer descriptor expects). Loads past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Asynchronous copy of `rows` (multiple of 16) rows of 64 bytes from a buffer resource
// into a swizzled LDS tile, without staging through registers (buffer_load ... lds). Rows
// past the resource's range arrive as zeros. Wave w of nw issues instructions w, w + nw,
// ...; each instruction fills 16 rows (1 KB; lane l -> row l/4, slot l%4).
__device__ __forceinline__ void stage_rows(__amdgpu_buffer_rsrc_t src, unsigned char* tile, int rows, int w, int nw,
                                           int lane) {
  for (int j = w; j < rows / 16; j += nw) {
    const int r = 16 * j + (lane >> 2);
    const int c = (lane & 3) ^ swz(r);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)(tile + 1024 * j), 16,
                                             r * 64 + 16 * c, 0, 0, 0);
  }
}

// Asynchronous copy of `rows` floats (a multiple of 64: every copy writes 64 lanes) from a
// buffer resource into LDS (zeros past its range).
__device__ __forceinline__ void stage_floats(__amdgpu_buffer_rsrc_t src, float* dst, int rows, int w, int nw,
                                             int lane) {
  for (int j = w; j < rows / 64; j += nw)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)(dst + 64 * j), 4,
                                             4 * (64 * j + lane), 0, 0, 0);
}

}  // namespace swin
