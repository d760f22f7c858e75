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

// Maximum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane rows at one position),
// with gfx950's row-swapping permutes instead of LDS round trips. Each swap of v with itself
// leaves, in its two results, a lane's own value and its partner's (across the 32-lane halves,
// then across adjacent rows), so the maximum of the two results is the pairwise maximum.
__device__ __forceinline__ float wave_max_xor16_32(float v) {
  const auto h = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                                  false, false);
  v = fmaxf(__builtin_bit_cast(float, (unsigned)h[0]), __builtin_bit_cast(float, (unsigned)h[1]));
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float wave_sum_xor16_32(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
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

// Lanes l and l ^ 16 (g = l / 16 and g ^ 1, same l % 16) hold columns 4 g .. 4 g + 3 of one
// row in v0 and columns 16 + 4 g .. 16 + 4 g + 3 in v1. After one exchange an even-g lane
// holds columns 4 g .. 4 g + 7 and an odd-g lane columns 4 g + 12 .. 4 g + 19 (both start at
// pair_col(g)), so each lane writes one 16-byte piece and four lanes a whole 64-byte row piece.
// Every lane of the wave must take part.
__device__ __forceinline__ bf16x8 pair_cols(bf16x4 v0, bf16x4 v1, int g) {
  const bool even = (g & 1) == 0;
  const u32x2 send = __builtin_bit_cast(u32x2, even ? v1 : v0);
  u32x2 recv;
  recv[0] = (uint32_t)__shfl_xor((int)send[0], 16);
  recv[1] = (uint32_t)__shfl_xor((int)send[1], 16);
  const bf16x4 r = __builtin_bit_cast(bf16x4, recv);
  return even ? bf16x8{v0[0], v0[1], v0[2], v0[3], r[0], r[1], r[2], r[3]}
              : bf16x8{r[0], r[1], r[2], r[3], v1[0], v1[1], v1[2], v1[3]};
}
__device__ __forceinline__ int pair_col(int g) { return (g & 1) == 0 ? 4 * g : 4 * g + 12; }

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

// (float)h - x for the low or high fp16 half h of a packed pair, in one mixed-precision FMA
// (the compiler emits a conversion and a subtraction for the plain expression).
__device__ __forceinline__ float half_lo_minus(uint32_t pair, float x) {
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(x));
  return r;
}
__device__ __forceinline__ float half_hi_minus(uint32_t pair, float x) {
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(x));
  return r;
}

// LDS byte address of a pointer into a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// The two V^T-style MFMA operands of a swizzled tile (see tile_frag_tr) for columns
// col0 + li and col0 + 16 + li, from the lane offsets off0 = swz_off(r, col) and
// off1 = swz_off(r, col + 16) of its row r = row0 + 4 g + li/4 (rows r and r + 16 share a
// swizzle, so the second read of each pair is 1 KB further). The four transposing reads are
// inline assembly ended by their own LDS wait, so the compiler adds no vector-memory wait in
// front of them: kernels that keep direct-to-LDS copies to other buffers in flight across
// these reads order those copies themselves.
__device__ __forceinline__ void tile_frag_tr2_at(const unsigned char* tile, int off0, int off1, bf16x8& f0,
                                                 bf16x8& f1) {
  const uint32_t base = lds_addr(tile);
  const uint32_t a0 = base + off0, a2 = base + off1;
  u32x2 v0, v1, v2, v3;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:1024\n\t"
      "ds_read_b64_tr_b16 %2, %5\n\t"
      "ds_read_b64_tr_b16 %3, %5 offset:1024\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
      : "v"(a0), "v"(a2)
      : "memory");
  const bf16x4 lo0 = __builtin_bit_cast(bf16x4, v0), hi0 = __builtin_bit_cast(bf16x4, v1);
  const bf16x4 lo1 = __builtin_bit_cast(bf16x4, v2), hi1 = __builtin_bit_cast(bf16x4, v3);
  f0 = bf16x8{lo0[0], lo0[1], lo0[2], lo0[3], hi0[0], hi0[1], hi0[2], hi0[3]};
  f1 = bf16x8{lo1[0], lo1[1], lo1[2], lo1[3], hi1[0], hi1[1], hi1[2], hi1[3]};
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

// Asynchronous 16-byte-per-lane copy from global memory (a 64-bit address per lane) into
// LDS: lane l writes bytes [16 l, 16 l + 16) of the 1 KB at lds_base (wave-uniform).
__device__ __forceinline__ void lds_copy16(const void* src, unsigned char* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// s_waitcnt vmcnt(n) for a wave-uniform n <= 15: wait until at most n vector-memory
// operations of this wave are outstanding (they complete in issue order).
__device__ __forceinline__ void vm_wait(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
    case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
  }
}

}  // namespace swin
