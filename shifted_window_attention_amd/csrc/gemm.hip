// bf16 MFMA GEMMs of the attention module (fp32 accumulation).
//
//   k_gemm_nt:   C[m, n] = sum_k A[m, k] * B[n, k]   (both operands K-contiguous)
//                A rows may be gathered through a row map (the cyclic shift + window
//                partition fused into the operand load), and the epilogue writes
//                head-split q/k/v planes or plain rows (optionally through a row map)
//                and can also form per-head row dot products with a second matrix.
//   k_gemm_nt_wide: the same product for the QKV projection and, at head_dim 32, for dO with
//                its per-head row dots (gathered A rows, head-split epilogue from registers)
//                on 256 x 256 tiles fed by direct global->LDS copies.
//   k_gemm_tn:   P[s, m, n] = sum_{t in chunk s} A[t, m] * B[t, n]   (contraction over
//                tokens for the weight gradients; deterministic split-K partials)
//   k_reduce_splits: fixed-order sum of the split-K partials (weights and biases).
//
// All run on v_mfma_f32_32x32x16_bf16. k_gemm_nt: 256 threads (4 waves of 64),
// 64-deep K steps staged through LDS via registers, rows padded by 16 bytes so that both
// the row-wise 16-byte stores and the MFMA fragment reads are bank-conflict free.
// k_gemm_tn: operand tiles copied straight into swizzled LDS tiles, double-buffered.
#include "device_common.h"
#include "swin_internal.h"

#include <type_traits>

namespace swin {

struct EpiParams {
  int mode;                  // 0: rows (optionally scattered), 1: head-split planes [P][nh][n_tok][hd],
                             // 2: rows of GELU(C + bias), with C + bias also written to out2,
                             // 3: rows of C * GELU'(aux) (aux [M][N] bf16, no bias)
  bf16* out;
  bf16* out2;                // mode 2: pre-activation rows [M][N]
  const bf16* aux;           // mode 3: the pre-activation the GELU derivative is taken at
  const bf16* res;           // mode 0: if set, residual rows added before rounding (same layout as out)
  const float* res_f32;      // mode 0: if set, fp32 residual rows added before rounding (pitch ldc)
  float* out_f32;            // mode 0: if set, the rows are written here in fp32 (pitch ldc) instead of to out
  const int32_t* out_rows;   // mode 0: destination row of each C row (NULL: identity)
  int64_t ldc;               // mode 0: row pitch of out (elements)
  const bf16* bias;          // [N] or NULL
  float qscale;              // mode 1: factor for columns < C (the q block)
  int C, nh, hd;
  int64_t n_tok;
  const bf16* dot_o;         // mode 1, one plane: if set, also write dot_out[head][m] = dot_scale *
  float* dot_out;            //   (sum over the head's columns of C[m, :] * dot_o[row(m), :])
  const int32_t* dot_rows;   //   with row(m) = dot_rows[m] (NULL: m)
  float dot_scale;
};

template <int BM, int BN>
struct NtCfg {
  static constexpr int NT = 256;
  static constexpr int BK = 64;
  static constexpr int PITCH = BK + 8;        // bf16 per LDS row of a K step
  static constexpr int WAVES_M = 2, WAVES_N = 2;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int A_CH = BM * BK / 8 / NT;  // 16-byte chunks per thread per K step
  static constexpr int B_CH = BN * BK / 8 / NT;
  static constexpr int CPITCH = BN + 8;        // bf16 per LDS row of the epilogue tile
  static constexpr int LDS_MAIN = (BM + BN) * PITCH;
  static constexpr int LDS_EPI = BM * CPITCH;
  static constexpr int LDS_ELEMS = LDS_MAIN > LDS_EPI ? LDS_MAIN : LDS_EPI;
};

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2. Remap the
// linear block id so that every XCD walks a contiguous range of tiles with the N tile
// fastest: the N tiles that reuse one block of gathered A rows then run back-to-back on
// the same XCD. Returns false for the padding blocks of the last round.
__device__ __forceinline__ bool xcd_tile(int64_t n_tiles, int nt, int64_t& mt_out, int& nt_out) {
  const int64_t b = blockIdx.x;
  const int64_t per = gridDim.x / 8;
  const int64_t logical = (b % 8) * per + b / 8;
  if (logical >= n_tiles) return false;
  mt_out = logical / nt;
  nt_out = (int)(logical % nt);
  return true;
}

static inline unsigned xcd_grid(int64_t n_tiles) { return (unsigned)((n_tiles + 7) / 8 * 8); }

// Exact GELU, a Phi(a), and its derivative Phi(a) + a phi(a). erf is evaluated with
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26 (|error| <= 1.5e-7
// for x >= 0, odd extension for x < 0), far below the bf16 rounding of the results; the
// factor exp(-x^2) of that formula at x = |a|/sqrt(2) is exp(-a^2/2), which also gives phi.
__device__ __forceinline__ void gelu_parts(float a, float& cdf, float& g) {
  const float z = fabsf(a) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.f));
  const float poly =
      t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f), -0.284496736f), 0.254829592f);
  g = __expf(-z * z);
  const float erf_abs = fmaf(-poly, g, 1.f);
  cdf = 0.5f + 0.5f * (a < 0.f ? -erf_abs : erf_abs);
}
__device__ __forceinline__ float gelu_f(float a) {
  float cdf, g;
  gelu_parts(a, cdf, g);
  return a * cdf;
}
__device__ __forceinline__ float gelu_grad_f(float a) {
  float cdf, g;
  gelu_parts(a, cdf, g);
  return fmaf(a * 0.39894228040143268f, g, cdf);
}

// Epilogue of the element-wise modes (2, 3, and 0 with a residual or an fp32 output): the accumulator tile
// plus bias goes through LDS as fp32 in two halves of BM/2 rows, so the residual add or the
// activation is applied before the single rounding to bf16; 16-byte row stores. The rows a
// thread reads (GELU pre-activation or residual) are loaded for the whole half before the
// LDS phase, so their latency overlaps it.
template <int BM, int BN>
__device__ __forceinline__ void epilogue_f32(const f32x16 (&acc)[NtCfg<BM, BN>::TM][NtCfg<BM, BN>::TN], bf16* smem,
                                             int tid, int lane, int wm, int wn, int64_t m0, int n0, int64_t M, int N,
                                             const EpiParams& ep) {
  using Cfg = NtCfg<BM, BN>;
  constexpr int HALF = BM / 2, FP = BN + 4;  // fp32 pitch
  static_assert(Cfg::WAVES_M == 2 && HALF == Cfg::WTM, "one wave row per half");
  static_assert(HALF * FP * 4 <= Cfg::LDS_ELEMS * 2, "an fp32 half tile fits the LDS of the main loop");
  float* Cs = (float*)smem;
  const int fr = lane & 31;
  constexpr int CH_PER_ROW = BN / 8;
  constexpr int ROW_STEP = Cfg::NT / CH_PER_ROW;
  constexpr int ITERS = HALF / ROW_STEP;
  static_assert(HALF % ROW_STEP == 0, "uniform copy-out loop");
  const int cc = (tid % CH_PER_ROW) * 8;
  const int n = n0 + cc;
  const int row0 = tid / CH_PER_ROW;
  const bf16* src = ep.mode == 3 ? ep.aux : (ep.mode == 0 ? ep.res : nullptr);
  for (int half = 0; half < 2; ++half) {
    bf16x8 pre[ITERS];
    if (src) {
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        const int64_t m = m0 + HALF * half + row0 + it * ROW_STEP;
        if (m < M && n < N) {
          const int64_t orow = (ep.mode == 0 && ep.out_rows) ? (int64_t)ep.out_rows[m] : m;
          pre[it] = *(const bf16x8*)(src + orow * ep.ldc + n);
        }
      }
    }
    if (wm == half) {
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j) {
        const int col = wn * Cfg::WTN + 32 * j + fr;
        const float bv = (ep.bias && n0 + col < N) ? to_f32(ep.bias[n0 + col]) : 0.f;
#pragma unroll
        for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            Cs[row * FP + col] = acc[i][j][r] + bv;
          }
      }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int row = row0 + it * ROW_STEP;
      const int64_t m = m0 + HALF * half + row;
      if (m >= M || n >= N) continue;
      const f32x4 lo = *(const f32x4*)(Cs + row * FP + cc), hi = *(const f32x4*)(Cs + row * FP + cc + 4);
      float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const int64_t orow = (ep.mode == 0 && ep.out_rows) ? (int64_t)ep.out_rows[m] : m;
      if (ep.mode == 0) {
        // residual rows (bf16 or fp32) join the fp32 value before its one rounding, or before
        // an fp32 store
        if (ep.res) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += to_f32(pre[it][e]);
        }
        if (ep.res_f32) {
          const float* r = ep.res_f32 + orow * ep.ldc + n;
          const f32x4 r0 = *(const f32x4*)r, r1 = *(const f32x4*)(r + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] += r0[e];
            v[4 + e] += r1[e];
          }
        }
        if (ep.out_f32) {
          float* dst = ep.out_f32 + orow * ep.ldc + n;
          *(f32x4*)dst = f32x4{v[0], v[1], v[2], v[3]};
          *(f32x4*)(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
          continue;
        }
      }
      bf16x8 o;
      if (ep.mode == 2) {
        bf16x8 pa;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pa[e] = to_bf16(v[e]);
          o[e] = to_bf16(gelu_f(v[e]));
        }
        *(bf16x8*)(ep.out2 + m * ep.ldc + n) = pa;
      } else if (ep.mode == 3) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = to_bf16(v[e] * gelu_grad_f(to_f32(pre[it][e])));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = to_bf16(v[e]);
      }
      *(bf16x8*)(ep.out + orow * ep.ldc + n) = o;
    }
    __syncthreads();
  }
}

template <int BM, int BN>
__global__ __launch_bounds__(256, BM == 128 ? 3 : 2) void k_gemm_nt(const bf16* __restrict__ A, int64_t lda,
                                                    const int32_t* __restrict__ a_rows,
                                                    const bf16* __restrict__ B, int64_t ldb, int64_t M, int N,
                                                    int K, EpiParams ep) {
  using Cfg = NtCfg<BM, BN>;
  __shared__ __attribute__((aligned(16))) bf16 smem[Cfg::LDS_ELEMS];
  bf16* As = smem;
  bf16* Bs = smem + BM * Cfg::PITCH;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  int64_t mt;
  int ntile;
  const int n_nt = (N + BN - 1) / BN;
  if (!xcd_tile(((M + BM - 1) / BM) * n_nt, n_nt, mt, ntile)) return;
  const int64_t m0 = mt * BM;
  const int n0 = ntile * BN;

  // per-thread source rows of the A and B chunks (clamped at the tails; clamped rows are
  // computed but never stored)
  const bf16* a_src[Cfg::A_CH];
  const bf16* b_src[Cfg::B_CH];
  const int c8 = (tid & 7) * 8;
#pragma unroll
  for (int i = 0; i < Cfg::A_CH; ++i) {
    int64_t r = m0 + (tid >> 3) + 32 * i;
    r = r < M ? r : M - 1;
    const int64_t g = a_rows ? (int64_t)a_rows[r] : r;
    a_src[i] = A + g * lda + c8;
  }
#pragma unroll
  for (int i = 0; i < Cfg::B_CH; ++i) {
    int r = n0 + (tid >> 3) + 32 * i;
    r = r < N ? r : N - 1;
    b_src[i] = B + (int64_t)r * ldb + c8;
  }

  f32x16 acc[Cfg::TM][Cfg::TN];
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) acc[i][j] = f32x16{};

  bf16x8 ra[Cfg::A_CH], rb[Cfg::B_CH];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < Cfg::A_CH; ++i) ra[i] = *(const bf16x8*)(a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < Cfg::B_CH; ++i) rb[i] = *(const bf16x8*)(b_src[i] + k0);
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < Cfg::A_CH; ++i) *(bf16x8*)(As + ((tid >> 3) + 32 * i) * Cfg::PITCH + c8) = ra[i];
#pragma unroll
    for (int i = 0; i < Cfg::B_CH; ++i) *(bf16x8*)(Bs + ((tid >> 3) + 32 * i) * Cfg::PITCH + c8) = rb[i];
  };

  const int KT = K / Cfg::BK;
  load(0);
  store();
  __syncthreads();
  const int fr = lane & 31;          // fragment row/column
  const int fk = (lane >> 5) * 8;    // fragment k offset
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) load((kt + 1) * Cfg::BK);
#pragma unroll
    for (int ks = 0; ks < Cfg::BK / 16; ++ks) {
      bf16x8 fa[Cfg::TM], fb[Cfg::TN];
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i)
        fa[i] = *(const bf16x8*)(As + (wm * Cfg::WTM + 32 * i + fr) * Cfg::PITCH + ks * 16 + fk);
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
        fb[j] = *(const bf16x8*)(Bs + (wn * Cfg::WTN + 32 * j + fr) * Cfg::PITCH + ks * 16 + fk);
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j) acc[i][j] = mfma32(fa[i], fb[j], acc[i][j]);
    }
    __syncthreads();
    if (kt + 1 < KT) {
      store();
      __syncthreads();
    }
  }

  if (ep.mode >= 2 || ep.res || ep.res_f32 || ep.out_f32) {
    epilogue_f32<BM, BN>(acc, smem, tid, lane, wm, wn, m0, n0, M, N, ep);
    return;
  }
  // epilogue: scale/bias in registers, bf16 tile through LDS, 16-byte row stores
  bf16* Cs = smem;
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const int col = wn * Cfg::WTN + 32 * j + fr;
    const int n = n0 + col;
    const float bv = (ep.bias && n < N) ? to_f32(ep.bias[n]) : 0.f;
    const float sc = (ep.mode == 1 && n < ep.C) ? ep.qscale : 1.f;
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * Cfg::WTM + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        Cs[row * Cfg::CPITCH + col] = to_bf16((acc[i][j][r] + bv) * sc);
      }
  }
  __syncthreads();
  // copy-out: a thread keeps one 8-column chunk and walks rows, so the column part of its
  // destination (plane, head and offset, or column) is computed once
  constexpr int CH_PER_ROW = BN / 8;
  constexpr int ROW_STEP = Cfg::NT / CH_PER_ROW;
  constexpr int ITERS = BM / ROW_STEP;
  static_assert(Cfg::NT % CH_PER_ROW == 0 && BM % ROW_STEP == 0, "uniform copy-out loop");
  const int cc = (tid % CH_PER_ROW) * 8;
  const int n = n0 + cc;
  const int row0 = tid / CH_PER_ROW;
  int64_t col_off, row_pitch;
  if (ep.mode == 1) {
    const int plane = n / ep.C;
    const int rem = n - plane * ep.C;
    const int head = rem / ep.hd;
    col_off = ((int64_t)plane * ep.nh + head) * ep.n_tok * ep.hd + (rem - head * ep.hd);
    row_pitch = ep.hd;
  } else {
    col_off = n;
    row_pitch = ep.ldc;
  }
  if (!ep.dot_o) {
#pragma unroll 4
    for (int it = 0; it < ITERS; ++it) {
      const int row = row0 + ROW_STEP * it;
      const int64_t m = m0 + row;
      if (m < M && n < N) {
        const int64_t orow = (ep.mode == 0 && ep.out_rows) ? (int64_t)ep.out_rows[m] : m;
        *(bf16x8*)(ep.out + col_off + orow * row_pitch) = *(const bf16x8*)(Cs + row * Cfg::CPITCH + cc);
      }
    }
  } else {
    // Row dot products with dot_o: every row's chunk of dot_o is loaded up front (the
    // accumulators are free by now), so the latency of those gathered loads is paid once.
    bf16x8 ov[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int64_t m = m0 + row0 + ROW_STEP * it;
      ov[it] = bf16x8{};
      if (m < M && n < N) {
        const int64_t drow = ep.dot_rows ? (int64_t)ep.dot_rows[m] : m;
        ov[it] = *(const bf16x8*)(ep.dot_o + drow * ep.C + n);
      }
    }
    const int64_t dot_head = (int64_t)(n / ep.hd) * ep.n_tok;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int row = row0 + ROW_STEP * it;
      const int64_t m = m0 + row;
      const bool valid = m < M && n < N;
      const bf16x8 v = *(const bf16x8*)(Cs + row * Cfg::CPITCH + cc);
      float dot = 0.f;
      if (valid) {
        const int64_t orow = (ep.mode == 0 && ep.out_rows) ? (int64_t)ep.out_rows[m] : m;
        *(bf16x8*)(ep.out + col_off + orow * row_pitch) = v;
#pragma unroll
        for (int e = 0; e < 8; ++e) dot += to_f32(v[e]) * to_f32(ov[it][e]);
      }
      // the hd/8 chunks of one (row, head) sit in hd/8 consecutive lanes (head_dim <= 128)
      for (int sh = 1; sh < ep.hd / 8; sh <<= 1) dot += __shfl_xor(dot, sh);
      if (valid && (tid & (ep.hd / 8 - 1)) == 0) ep.dot_out[dot_head + m] = dot * ep.dot_scale;
    }
  }
}

// ---------------------------------------------------------------------------
// Wide NT GEMM for the QKV projection: C = A B^T with 256 x 256 output tiles, 8 waves of
// 128 x 64 (v_mfma_f32_32x32x16_bf16), one workgroup per CU.
//
// Operands are copied straight into LDS (global_load_lds, 16 bytes per lane, gathered A rows
// allowed) through a ring of three 32-deep K stages of 32 KB, each 64-byte tile row holding
// its four 16-byte chunks at slot chunk ^ swz(row). The loop is software-pipelined across K
// steps: a step's first fragments are read before the step starts, and the barrier that makes
// the next stage visible sits after the step's last MFMAs are issued, so it overlaps their
// execution; right after that barrier the stage the step used takes the copies of the stage
// three ahead. The accumulators hold transposed 32 x 32 blocks (the MFMA's operands swapped),
// so a lane owns one output row and 4 consecutive columns per register group; the epilogue
// (bias, loaded before the loop, q scale, bf16) pairs lanes 32 apart and stores 16-byte row
// pieces straight from registers: in head-split planes (mode 1) the 32 rows of a block are 32
// consecutive 64-byte rows, so the stores are contiguous. (Plain rows, mode 0, are supported
// but not launched: on rows of a wide matrix the same stores are scattered, and the LDS-staged
// copy-out of k_gemm_nt measured faster there.) DOT (the proj backward at head_dim 32, where a
// 32-column block is one head): also -D = -rowsum(dO o) per head, from the lane's two stored
// pieces and the matching pieces of the gathered o row, in the 8-column chunk order of
// k_gemm_nt's reduction. Results are bitwise those of k_gemm_nt: the same products summed over
// K, and the same row dots, in the same order.
// ---------------------------------------------------------------------------
namespace wide {
constexpr int BM = 256, BN = 256, BK = 32, ST = 3;
constexpr int NW = 8, NT = 64 * NW, WN = 4;   // waves: 2 along M, 4 along N
constexpr int WTM = 128, WTN = 64, TM = WTM / 32, TN = WTN / 32;
constexpr int A_BYTES = BM * 64, STAGE = (BM + BN) * 64;  // one 32-deep K step of A and B
constexpr int CP = BM / 16 / NW + BN / 16 / NW;           // 1 KB copies per wave per stage
constexpr int LDS = ST * STAGE;

__device__ __forceinline__ bf16x8 frag(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
  return __builtin_bit_cast(bf16x8, v);
}
template <int NA, int NB>
__device__ __forceinline__ void wait_frags(bf16x8 (&fa)[NA], bf16x8 (&fb)[NB]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < NA; ++i) asm volatile("" : "+v"(fa[i]));
#pragma unroll
  for (int j = 0; j < NB; ++j) asm volatile("" : "+v"(fb[j]));
}
// Lanes 0-31 of y trade places with lanes 32-63 of x. Inline assembly: the instruction writes
// both of its registers, and the compiler's builtin for it has been seen to read one result
// register twice when both results feed one expression; the s_nop gives the wait states a VALU
// write needs before the swap reads the register.
__device__ __forceinline__ void permlane32_swap(uint32_t& x, uint32_t& y) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void swap_upper_lower(bf16x4& x, bf16x4& y) {
  u32x2 xv = __builtin_bit_cast(u32x2, x), yv = __builtin_bit_cast(u32x2, y);
  uint32_t x0 = xv[0], x1 = xv[1], y0 = yv[0], y1 = yv[1];
  permlane32_swap(x0, y0);
  permlane32_swap(x1, y1);
  x = __builtin_bit_cast(bf16x4, u32x2{x0, x1});
  y = __builtin_bit_cast(bf16x4, u32x2{y0, y1});
}
__device__ __forceinline__ bf16x8 join8(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// this wave's copies of a stage have landed once at most `newer` later stages' are in flight
__device__ __forceinline__ void wait_stage(int newer) {
  if (newer >= 2)
    vm_wait(2 * CP);
  else if (newer == 1)
    vm_wait(CP);
  else
    vm_wait(0);
}
}  // namespace wide

template <bool DOT>
__global__ __launch_bounds__(wide::NT, 1) void k_gemm_nt_wide(const bf16* __restrict__ A, int64_t lda,
                                                             const int32_t* __restrict__ a_rows,
                                                             const bf16* __restrict__ B, int64_t ldb, int64_t M,
                                                             int N, int K, EpiParams ep) {
  using namespace wide;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / WN, wn = w % WN;
  int64_t mt;
  int ntile;
  const int n_nt = (N + BN - 1) / BN;
  if (!xcd_tile(((M + BM - 1) / BM) * n_nt, n_nt, mt, ntile)) return;
  const int64_t m0 = mt * BM;
  const int n0 = ntile * BN;

  // copy q of this wave fills tile rows 16 (w + NW q) + lane/4 at slot lane%4, i.e. logical
  // chunk (lane%4) ^ swz(row); rows past M or N repeat the last row (computed, never stored)
  const unsigned char* a_src[BM / 16 / NW];
  const unsigned char* b_src[BN / 16 / NW];
#pragma unroll
  for (int q = 0; q < BM / 16 / NW; ++q) {
    const int r = 16 * (w + NW * q) + (lane >> 2);
    int64_t gr = m0 + r;
    gr = gr < M ? gr : M - 1;
    if (a_rows) gr = a_rows[gr];
    a_src[q] = (const unsigned char*)(A + gr * lda) + 16 * ((lane & 3) ^ swz(r));
  }
#pragma unroll
  for (int q = 0; q < BN / 16 / NW; ++q) {
    const int r = 16 * (w + NW * q) + (lane >> 2);
    int64_t gr = n0 + r;
    gr = gr < N ? gr : N - 1;
    b_src[q] = (const unsigned char*)(B + gr * ldb) + 16 * ((lane & 3) ^ swz(r));
  }
  auto issue = [&](int kt) {
    unsigned char* st = smem + (kt % ST) * STAGE;
    const int kb = kt * 64;
#pragma unroll
    for (int q = 0; q < BM / 16 / NW; ++q) lds_copy16(a_src[q] + kb, st + 1024 * (w + NW * q));
#pragma unroll
    for (int q = 0; q < BN / 16 / NW; ++q) lds_copy16(b_src[q] + kb, st + A_BYTES + 1024 * (w + NW * q));
  };

  // fragment offsets: A rows wm WTM + 32 i + lane%32, B rows wn WTN + 32 j + lane%32, chunk
  // lane/32 (K slice 0) or 2 + lane/32 (slice 1); rows 32 apart share their swizzle
  const int fr = lane & 31;
  const uint32_t l0 = (uint32_t)(fr * 64 + 16 * ((lane >> 5) ^ swz(fr)));
  const uint32_t l1 = (uint32_t)(fr * 64 + 16 * (((lane >> 5) | 2) ^ swz(fr)));
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t a_w = (uint32_t)(wm * WTM * 64), b_w = (uint32_t)(A_BYTES + wn * WTN * 64);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  // the bias of the lane's 4-column groups, and the dot_o rows of its output rows, loaded here
  // so that their latency hides behind the loop
  const int half = lane >> 5;
  bf16x4 bias4[TN][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const int n = n0 + wn * WTN + 32 * j + 8 * gg + 4 * half;
      bias4[j][gg] = (ep.bias && n < N) ? *(const bf16x4*)(ep.bias + n) : bf16x4{};
    }
  int drow[TM];
  if constexpr (DOT) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      int64_t m = m0 + wm * WTM + 32 * i + fr;
      m = m < M ? m : M - 1;
      drow[i] = ep.dot_rows ? ep.dot_rows[m] : (int)m;
    }
  }

  const int KT = K / BK;
#pragma unroll
  for (int s = 0; s < ST; ++s)
    if (s < KT) issue(s);
  wait_stage((ST - 1 < KT - 1 ? ST - 1 : KT - 1));  // stage 0 (the stages issued after it may fly)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  bf16x8 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) fa0[i] = frag(lds0 + a_w + l0 + 2048 * i);
#pragma unroll
  for (int j = 0; j < TN; ++j) fb0[j] = frag(lds0 + b_w + l0 + 2048 * j);
  for (int kt = 0; kt < KT; ++kt) {
    const uint32_t sb = lds0 + (uint32_t)((kt % ST) * STAGE);
    wait_frags(fa0, fb0);
#pragma unroll
    for (int i = 0; i < TM; ++i) fa1[i] = frag(sb + a_w + l1 + 2048 * i);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb1[j] = frag(sb + b_w + l1 + 2048 * j);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(fb0[j], fa0[i], acc[i][j]);
    wait_frags(fa1, fb1);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(fb1[j], fa1[i], acc[i][j]);
    if (kt + 1 < KT) {
      // the newest stage issued so far is kt - 1 + ST (or KT - 1)
      const int last = kt - 1 + ST < KT - 1 ? kt - 1 + ST : KT - 1;
      wait_stage(last - (kt + 1));
      // every wave's copies of stage kt+1 have landed and every wave has read stage kt
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (kt + ST < KT) issue(kt + ST);  // into the buffer step kt used
      const uint32_t sn = lds0 + (uint32_t)(((kt + 1) % ST) * STAGE);
#pragma unroll
      for (int i = 0; i < TM; ++i) fa0[i] = frag(sn + a_w + l0 + 2048 * i);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb0[j] = frag(sn + b_w + l0 + 2048 * j);
    }
  }

  // epilogue: bias and q scale on the transposed blocks (a lane's row and 4 consecutive columns
  // per register group g), bf16; lanes 32 apart then trade groups so that each lane holds 8
  // consecutive columns twice (columns 8 half .. +7 and 16 + 8 half .. +7 of the 32-column
  // block) and stores them straight to its row as two 16-byte pieces: the 32 rows of a block
  // are consecutive rows of one head plane (mode 1), so every row piece of the block is
  // written by one pair of stores, with no pass through LDS
  // row dot products (head_dim 32: a 32-column block is one head): the dot_o pieces that match
  // the lane's stored pieces, for all its rows and blocks, loaded before any is used
  bf16x8 ovall[TN][TM][2];
  if constexpr (DOT) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int pc = 0; pc < 2; ++pc)
          ovall[j][i][pc] = *(const bf16x8*)(ep.dot_o + (int64_t)drow[i] * ep.C + n0 + wn * WTN + 32 * j + 16 * pc + 8 * half);
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int nblk = n0 + wn * WTN + 32 * j;
    const float scv = (ep.mode == 1 && nblk < ep.C) ? ep.qscale : 1.f;  // C is a multiple of 32
    int64_t col_off[2], row_pitch;
#pragma unroll
    for (int pc = 0; pc < 2; ++pc) {
      const int n = nblk + 16 * pc + 8 * half;
      if (ep.mode == 1) {
        const int plane = n / ep.C;
        const int rem = n - plane * ep.C;
        const int head = rem / ep.hd;
        col_off[pc] = ((int64_t)plane * ep.nh + head) * ep.n_tok * ep.hd + (rem - head * ep.hd);
      } else {
        col_off[pc] = n;
      }
    }
    row_pitch = ep.mode == 1 ? ep.hd : ep.ldc;
    bf16x8 (&ov)[TM][2] = ovall[j];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      bf16x4 c[4];
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
#pragma unroll
        for (int e = 0; e < 4; ++e) c[gg][e] = to_bf16((acc[i][j][4 * gg + e] + to_f32(bias4[j][gg][e])) * scv);
      swap_upper_lower(c[0], c[1]);
      swap_upper_lower(c[2], c[3]);
      const bf16x8 p0 = join8(c[0], c[1]), p1 = join8(c[2], c[3]);
      const int64_t m = m0 + wm * WTM + 32 * i + fr;
      if (m < M) {
        const int64_t orow = (ep.mode == 0 && ep.out_rows) ? (int64_t)ep.out_rows[m] : m;
        const int n = nblk + 8 * half;
        if (n < N) *(bf16x8*)(ep.out + col_off[0] + orow * row_pitch) = p0;
        if (n + 16 < N) *(bf16x8*)(ep.out + col_off[1] + orow * row_pitch) = p1;
      }
      if constexpr (DOT) {
        // 8-column sums s0..s3 in column order (this lane: s0, s2 or s1, s3), combined as
        // (s0 + s1) + (s2 + s3): the order of the 8-column chunks' pairwise reduction
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a += to_f32(p0[e]) * to_f32(ov[i][0][e]);
#pragma unroll
        for (int e = 0; e < 8; ++e) b += to_f32(p1[e]) * to_f32(ov[i][1][e]);
        // lanes 0-31: (s0, s1); lanes 32-63: (s2, s3); then lanes 0-31 take the other half's sum
        uint32_t ua = __builtin_bit_cast(uint32_t, a), ub = __builtin_bit_cast(uint32_t, b);
        permlane32_swap(ua, ub);
        const float t = __builtin_bit_cast(float, ua) + __builtin_bit_cast(float, ub);
        uint32_t tx = __builtin_bit_cast(uint32_t, t), ty = tx;
        permlane32_swap(tx, ty);
        const float dot = t + __builtin_bit_cast(float, ty);
        if (half == 0 && m < M) ep.dot_out[(int64_t)(nblk / 32) * ep.n_tok + m] = dot * ep.dot_scale;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Weight-gradient GEMM: P[s] = sum over the tokens t of chunk s of A[t, m0:m0+256]^T B[t, n0:n0+256]
// (both operands token-major: a contraction over tokens), stored per split as
// P[s][m/4][n][m%4] so that each lane's four consecutive MFMA rows are one 16-byte store.
//
// 256 x 256 output tile, 8 waves of 128 x 64 (v_mfma_f32_32x32x16_bf16, 128 accumulators
// per lane), 64-token steps. Both 64 x 256 operand tiles are copied straight into LDS
// (buffer_load ... lds, no staging registers), double-buffered so step k+1 is in flight
// while step k is computed. The copy's buffer range ends at the chunk's last token, so the
// token tail arrives as zeros. The MFMA fragments need 8 consecutive tokens at one column:
// gfx950's transposing LDS read returns them from the token-major tile. Within each 512-byte
// tile row, 16-byte chunk c is stored at slot c ^ 4 (r & 3), which puts the 4 rows x 2
// chunks that one 16-lane group reads, and the neighbouring group's, in 16 distinct banks.
//
// The LDS reads are inline assembly and the steps are ordered by explicit waits: the
// compiler cannot tell a read of one stage buffer from the copies in flight into the other,
// and with its own reads (or a __syncthreads) it waits for every copy, the next step's
// included, before each step's first read. Each step starts by waiting for this wave's
// copies of the step (issued a whole step earlier), then an LDS-only barrier, then issues
// the next step's copies into the other buffer; fragment reads of K slice ks+1 are in flight
// while slice ks multiplies.
//
// The bias gradients (A's column sums) come from the A fragments already in registers. The
// Q = min(column tiles, 4) workgroups of the first Q column tiles share them: workgroup t
// sums the 32-column fragments i with i % Q == t, so every column is summed by exactly one
// workgroup and the work is spread over them. Inside a workgroup the four waves that share
// a row of column blocks take one 16-token K slice each (two-term dot products with ones,
// 8 tokens of one column per lane); the four slice sums are combined through LDS in a
// fixed order.
// ---------------------------------------------------------------------------
namespace tn {
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NT = 512, NW = NT / 64;    // threads, waves
constexpr int WTM = 128, WTN = 64;       // per-wave tile
constexpr int ROWB = 512;                // bytes per tile row (256 bf16)
constexpr int TILEB = BK * ROWB;         // 32 KB per operand tile
constexpr int WN = BN / WTN;             // waves per row of column blocks = K slices per step
struct Stage {
  unsigned char a[TILEB], b[TILEB];
};
__device__ __forceinline__ int slot(int r, int c) { return c ^ (4 * (r & 3)); }
}  // namespace tn

// 32x32x16 fragment: 8 consecutive tokens k0 + 8 (g>>1) + 0..7 at column col0 + lane % 32
// (g = lane / 16, L = lane % 16). Its two transposing reads (token rows r and r + 4, where
// r = k0 + 8 (g>>1) + L/4) start at the lane's byte address in the tile; column block
// c32 = col0 / 32 puts logical chunk 4 c32 + lp (lp = 2 (g&1) + (L&3)/2) at slot
// 4 (c32 ^ (r&3)) + lp, so the address is tn_lane_off(lane) + 64 (c32 ^ (r&3)) + K offset.
// Issued without a wait: the caller waits (tn_wait) before the registers are used.
__device__ __forceinline__ uint32_t tn_lane_off(int lane) {
  const int g = lane >> 4, L = lane & 15;
  const int rl = 8 * (g >> 1) + (L >> 2);
  return (uint32_t)(rl * tn::ROWB + 16 * (2 * (g & 1) + ((L & 3) >> 1)) + 8 * (L & 1));
}
__device__ __forceinline__ int tn_lane_rr(int lane) { return ((lane & 15) >> 2) & 3; }  // (r & 3)

template <int OFF>
__device__ __forceinline__ bf16x8 tn_frag_issue(uint32_t addr) {
  u32x2 lo, hi;
  asm volatile("ds_read_b64_tr_b16 %0, %2 offset:%3\n\tds_read_b64_tr_b16 %1, %2 offset:%4"
               : "=&v"(lo), "=&v"(hi)
               : "v"(addr), "i"(OFF), "i"(OFF + 4 * tn::ROWB));
  const bf16x4 l = __builtin_bit_cast(bf16x4, lo), h = __builtin_bit_cast(bf16x4, hi);
  return bf16x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
}

// Waits for this wave's LDS reads and ties the registers to the wait, so that no use of them
// is scheduled before it.
template <int NA, int NB>
__device__ __forceinline__ void tn_wait(bf16x8 (&fa)[NA], bf16x8 (&fb)[NB]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < NA; ++i) asm volatile("" : "+v"(fa[i]));
#pragma unroll
  for (int j = 0; j < NB; ++j) asm volatile("" : "+v"(fb[j]));
}

// Copy rows [0, 64) x 256 columns of a token-major operand (row pitch ld elements) starting
// at `base` into a swizzled tile. The buffer range ends after column `cols` of row valid - 1
// (the operand's last element when that row is its last), so rows past `valid` and that
// row's columns past `cols` arrive as zeros and no copy reads past the operand. Earlier
// rows' columns past `cols` hold the next row's values; they only feed outputs that are
// never stored. Wave w issues 4 of the 32 one-kilobyte copies (2 rows each; lane l -> row
// 2j + l/32, slot l%32).
__device__ __forceinline__ void tn_stage(const bf16* base, int64_t ld, int valid, int cols, unsigned char* tile,
                                         int w, int lane) {
  const uint32_t bytes = (uint32_t)(((int64_t)(valid - 1) * ld + cols) * 2);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, bytes);
#pragma unroll
  for (int i = 0; i < 32 / tn::NW; ++i) {
    const int j = w + tn::NW * i;
    const int r = 2 * j + (lane >> 5);
    const int c = tn::slot(r, lane & 31);  // slot lane%32 holds logical chunk slot ^ 4(r&3)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(tile + 1024 * j), 16,
                                             (uint32_t)(r * ld * 2 + 16 * c), 0, 0, 0);
  }
}

__global__ __launch_bounds__(tn::NT, 1) void k_gemm_tn(const bf16* __restrict__ A, int64_t lda,
                                                       const bf16* __restrict__ B, int64_t ldb, int64_t T, int M,
                                                       int N, int64_t chunk, int n_splits,
                                                       float* __restrict__ part, float* __restrict__ dbpart) {
  __shared__ __attribute__((aligned(1024))) tn::Stage stg[2];
  __shared__ float colsum[tn::WN][tn::BM];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  // tile order: N tile fastest, then M tile, then split (XCD-aware, see xcd_tile)
  const int n_nt = (N + tn::BN - 1) / tn::BN, n_mt = (M + tn::BM - 1) / tn::BM;
  int64_t ms;
  int ntile;
  if (!xcd_tile((int64_t)n_mt * n_nt * n_splits, n_nt, ms, ntile)) return;
  const int m0 = (int)(ms % n_mt) * tn::BM, n0 = ntile * tn::BN;
  const int s = (int)(ms / n_mt);
  const int64_t t_begin = (int64_t)s * chunk;
  const int64_t t_end = t_begin + chunk < T ? t_begin + chunk : T;
  const int steps = t_end > t_begin ? (int)((t_end - t_begin + tn::BK - 1) / tn::BK) : 0;

  constexpr int TM = tn::WTM / 32, TN = tn::WTN / 32;
  const int db_q = n_nt < TM ? n_nt : TM;       // workgroups sharing the column sums
  const bool do_db = dbpart != nullptr && ntile < db_q;
  const auto db_mine = [&](int i) { return i % db_q == ntile; };  // fragment i's columns here
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};
  float csum[TM] = {};  // column sums of K slice wn of every step, per A fragment

  // lane byte offsets of the fragments in stage 0 (stage 1 is one Stage further)
  const uint32_t lane_off = tn_lane_off(lane), rr = (uint32_t)tn_lane_rr(lane);
  uint32_t a_off[TM], b_off[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a_off[i] = lane_off + 64 * ((uint32_t)(wm * TM + i) ^ rr);
#pragma unroll
  for (int j = 0; j < TN; ++j) b_off[j] = lane_off + 64 * ((uint32_t)(wn * TN + j) ^ rr) + (uint32_t)tn::TILEB;
  const uint32_t st_base = lds_addr(&stg[0]);

  auto stage = [&](int k, tn::Stage& st) {
    const int64_t t0 = t_begin + (int64_t)k * tn::BK;
    const int valid = (int)(t_end - t0 < tn::BK ? t_end - t0 : tn::BK);
    tn_stage(A + t0 * lda + m0, lda, valid, M - m0 < tn::BM ? M - m0 : tn::BM, st.a, wave, lane);
    tn_stage(B + t0 * ldb + n0, ldb, valid, N - n0 < tn::BN ? N - n0 : tn::BN, st.b, wave, lane);
  };
  // fragments of K slice KS (16 tokens) of the stage at LDS address sb
  auto issue = [&](uint32_t sb, auto ks, bf16x8 (&fa)[TM], bf16x8 (&fb)[TN]) {
    constexpr int OFF = 16 * decltype(ks)::value * tn::ROWB;
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = tn_frag_issue<OFF>(sb + a_off[i]);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = tn_frag_issue<OFF>(sb + b_off[j]);
  };
  auto mma = [&](const bf16x8 (&fa)[TM], const bf16x8 (&fb)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(fa[i], fb[j], acc[i][j]);
  };
  static_assert(tn::BK == 64 && tn::WN == tn::BK / 16, "four K slices per step, one per column-block wave");
  const bf16x2 ones2 = {(bf16)1.f, (bf16)1.f};
  // bias gradients: the wave whose column-block index is KS adds the 8 tokens of each A
  // fragment of slice KS (column wm * WTM + 32 i + lane % 32, token half lane / 32)
  auto db_add = [&](auto ks, const bf16x8 (&fa)[TM]) {
    if (do_db && wn == decltype(ks)::value) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        if (db_mine(i)) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            csum[i] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{fa[i][2 * e], fa[i][2 * e + 1]}, ones2, csum[i], false);
        }
    }
  };

  if (steps > 0) stage(0, stg[0]);
  for (int k = 0; k < steps; ++k) {
    // this wave's copies of step k (issued a step ago) have landed; after the barrier every
    // wave's have, and every wave is done reading the buffer the next copies go to
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (k + 1 < steps) stage(k + 1, stg[(k + 1) & 1]);
    const uint32_t sb = st_base + (uint32_t)((k & 1) * sizeof(tn::Stage));
    bf16x8 f0a[TM], f0b[TN], f1a[TM], f1b[TN];
    using K0 = std::integral_constant<int, 0>;
    using K1 = std::integral_constant<int, 1>;
    using K2 = std::integral_constant<int, 2>;
    using K3 = std::integral_constant<int, 3>;
    issue(sb, K0{}, f0a, f0b);
    tn_wait(f0a, f0b);
    issue(sb, K1{}, f1a, f1b);
    mma(f0a, f0b);
    db_add(K0{}, f0a);
    tn_wait(f1a, f1b);
    issue(sb, K2{}, f0a, f0b);
    mma(f1a, f1b);
    db_add(K1{}, f1a);
    tn_wait(f0a, f0b);
    issue(sb, K3{}, f1a, f1b);
    mma(f0a, f0b);
    db_add(K2{}, f0a);
    tn_wait(f1a, f1b);
    mma(f1a, f1b);
    db_add(K3{}, f1a);
  }

  // partial tile as P[s][m/4][n][m%4]: a lane's 4 consecutive rows m of one column n are one
  // 16-byte store, and the split reduction reads them back as one 16-byte load (M % 4 == 0)
  float* P = part + (int64_t)s * M * N;
  const int fr = lane & 31;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * tn::WTN + 32 * j + fr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + wm * tn::WTM + 32 * i + 8 * q + 4 * (lane >> 5);
        if (n < N && m < M) {
          const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          *(f32x4*)(P + ((int64_t)(m >> 2) * N + n) * 4) = v;
        }
      }
    }
  if (do_db) {
    // the two token halves of a column (lanes l and l ^ 32), then the four K slices in order
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const float v = csum[i] + __shfl_xor(csum[i], 32);
      if (lane < 32) colsum[wn][wm * tn::WTM + 32 * i + lane] = v;
    }
    __syncthreads();
    if (tid < tn::BM && m0 + tid < M && db_mine((tid % tn::WTM) / 32)) {
      float v = 0.f;
      for (int q = 0; q < tn::WN; ++q) v += colsum[q][tid];  // fixed order
      dbpart[(int64_t)s * M + m0 + tid] = v;
    }
  }
}

// sum over k < S of rows[k * stride + t] (f32x4 units) in order of k; the loads are issued
// eight at a time ahead of their adds, so that they overlap
__device__ __forceinline__ f32x4 sum_rows(const float* rows, int64_t t, int64_t stride, int S) {
  constexpr int U = 8;
  const f32x4* src = (const f32x4*)rows + t;
  f32x4 acc = src[0];
  int k = 1;
  for (; k + U <= S; k += U) {
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[(k + u) * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc += v[u];
  }
  for (; k < S; ++k) acc += src[k * stride];
  return acc;
}

// Split-K reduction of the weight gradients, in order of s:
//   dw[m][n] = sum_s P[s][m/4][n][m%4]   (threads 0 .. M N / 4 - 1: 4 rows of one column)
//   db[m]    = sum_s dbpart[s][m]        (the next M / 4 threads: 4 consecutive entries)
__global__ __launch_bounds__(256) void k_reduce_splits(const float* __restrict__ part, int S, int M, int N,
                                                       float* __restrict__ dw, const float* __restrict__ dbpart,
                                                       float* __restrict__ db) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n_w = (int64_t)M * N / 4;
  if (t < n_w) {
    const int64_t mq = t / N;
    const int n = (int)(t - mq * N);
    const f32x4 acc = sum_rows(part, t, n_w, S);  // one split is n_w f32x4
    float* o = dw + (4 * mq) * N + n;
    o[0] = acc[0];
    o[N] = acc[1];
    o[2 * N] = acc[2];
    o[3 * N] = acc[3];
  } else if (db && t < n_w + M / 4) {
    const int64_t i = t - n_w;
    const f32x4 acc = sum_rows(dbpart, i, M / 4, S);
    float* o = db + 4 * i;  // the caller's pointer: no alignment beyond 4 bytes assumed
    o[0] = acc[0];
    o[1] = acc[1];
    o[2] = acc[2];
    o[3] = acc[3];
  }
}

// out[c][r] = in[r][c] for an R x Cn bf16 matrix.
__global__ void k_transpose_bf16(const bf16* __restrict__ in, bf16* __restrict__ out, int R, int Cn) {
  __shared__ bf16 tile[32][33];
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 256 threads: 32 x 8
  for (int k = ty; k < 32; k += 8) {
    const int r = r0 + k, c = c0 + tx;
    if (r < R && c < Cn) tile[k][tx] = in[(int64_t)r * Cn + c];
  }
  __syncthreads();
  for (int k = ty; k < 32; k += 8) {
    const int c = c0 + k, r = r0 + tx;
    if (r < R && c < Cn) out[(int64_t)c * R + r] = tile[tx][k];
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static hipError_t gemm_nt(const bf16* A, int64_t lda, const int32_t* a_rows, const bf16* B, int64_t ldb, int64_t M,
                          int N, int K, const EpiParams& ep, hipStream_t s) {
  if (ep.dot_o || K < 256) {
    // the row-dot epilogue holds a whole column of dot_o chunks per thread: 128-row tiles keep
    // three workgroups per CU (measured faster than 256 x 128 for this epilogue); so do
    // products of fewer than four 64-deep K steps, whose tiles are mostly set-up and epilogue
    // (C = 192: 5-6% faster; at K = 256 the larger tile is faster)
    constexpr int BM = 128, BN = 128;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    k_gemm_nt<BM, BN><<<xcd_grid(tiles), 256, 0, s>>>(A, lda, a_rows, B, ldb, M, N, K, ep);
  } else {
    constexpr int BM = 256, BN = 128;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    k_gemm_nt<BM, BN><<<xcd_grid(tiles), 256, 0, s>>>(A, lda, a_rows, B, ldb, M, N, K, ep);
  }
  return hipGetLastError();
}

hipError_t launch_qkv_fwd_bf16(const swin_attn_plan* p, const void* x, const void* w, const void* b, void* qkv,
                               hipStream_t s) {
  EpiParams ep{};
  ep.mode = 1;
  ep.out = (bf16*)qkv;
  ep.bias = (const bf16*)b;
  ep.qscale = p->tau * kLog2e;  // q is stored pre-scaled so that logits come out in log2 units
  ep.C = p->C;
  ep.nh = p->nh;
  ep.hd = p->hd;
  ep.n_tok = p->n_tok;
  // the wide kernel (K in 32-deep steps; C is a multiple of 64) when its 256-column tiles
  // divide 3C; otherwise the 128-column tiles waste less (measured equal or faster there)
  if ((3 * p->C) % wide::BN != 0)
    return gemm_nt((const bf16*)x, p->C, p->dev.perm, (const bf16*)w, p->C, p->n_tok, 3 * p->C, p->C, ep, s);
  const int64_t tiles = ((p->n_tok + wide::BM - 1) / wide::BM) * ((3 * p->C + wide::BN - 1) / wide::BN);
  k_gemm_nt_wide<false><<<xcd_grid(tiles), wide::NT, 0, s>>>((const bf16*)x, p->C, p->dev.perm, (const bf16*)w, p->C,
                                                       p->n_tok, 3 * p->C, p->C, ep);
  return hipGetLastError();
}

hipError_t launch_proj_fwd_bf16(const swin_attn_plan* p, const void* o, const void* w, const void* b, void* y,
                                hipStream_t s) {
  EpiParams ep{};
  ep.mode = 0;
  ep.out = (bf16*)y;  // o is in grid order already (the attention kernel put rows back)
  ep.ldc = p->C;
  ep.bias = (const bf16*)b;
  ep.qscale = 1.f;
  ep.C = p->C;
  return gemm_nt((const bf16*)o, p->C, nullptr, (const bf16*)w, p->C, p->n_tok, p->C, p->C, ep, s);
}

// Backward GEMM pieces, used by the backward driver.
hipError_t launch_dproj_bf16(const swin_attn_plan* p, const void* dy, const void* wprojT, void* dO, const void* o,
                             float* dd, hipStream_t s) {
  EpiParams ep{};
  ep.mode = 1;  // head-split, one plane, plus -D = -rowsum(dO * O) per head
  ep.out = (bf16*)dO;
  ep.dot_o = (const bf16*)o;
  ep.dot_rows = p->dev.perm;  // o is in grid order
  ep.dot_out = dd;
  ep.dot_scale = -1.f;        // the attention backward starts its dP products from -D
  ep.qscale = 1.f;
  ep.C = p->C;
  ep.nh = p->nh;
  ep.hd = p->hd;
  ep.n_tok = p->n_tok;
  // head_dim 32 with 256-column tiles dividing C: the wide kernel, whose register epilogue forms
  // each head's dot from the lane pair's pieces (a 32-column block is one head)
  if (p->hd != 32 || p->C % wide::BN != 0)
    return gemm_nt((const bf16*)dy, p->C, p->dev.perm, (const bf16*)wprojT, p->C, p->n_tok, p->C, p->C, ep, s);
  const int64_t tiles = ((p->n_tok + wide::BM - 1) / wide::BM) * (p->C / wide::BN);
  k_gemm_nt_wide<true><<<xcd_grid(tiles), wide::NT, 0, s>>>((const bf16*)dy, p->C, p->dev.perm, (const bf16*)wprojT,
                                                       p->C, p->n_tok, p->C, p->C, ep);
  return hipGetLastError();
}

hipError_t launch_dgrad_qkv_bf16(const swin_attn_plan* p, const void* dqkv, const void* wqkvT, void* dx,
                                 float* dx32, hipStream_t s) {
  EpiParams ep{};
  ep.mode = 0;
  ep.out = (bf16*)dx;  // dqkv is in grid order already
  ep.out_f32 = dx32;   // if set, dx goes there in fp32 instead
  ep.ldc = p->C;
  ep.qscale = 1.f;
  ep.C = p->C;
  return gemm_nt((const bf16*)dqkv, 3 * p->C, nullptr, (const bf16*)wqkvT, 3 * p->C, p->n_tok, p->C, 3 * p->C, ep,
                 s);
}

// The block's h = x + proj(o) in fp32: the projection's rows plus the bf16 residual x, stored
// without rounding (the block keeps its residual stream in fp32).
hipError_t launch_proj_fwd_res_f32(const swin_attn_plan* p, const void* o, const void* w, const void* b,
                                   const void* res, float* h, hipStream_t s) {
  EpiParams ep{};
  ep.mode = 0;
  ep.out_f32 = h;
  ep.res = (const bf16*)res;
  ep.ldc = p->C;
  ep.bias = (const bf16*)b;
  ep.qscale = 1.f;
  ep.C = p->C;
  return gemm_nt((const bf16*)o, p->C, nullptr, (const bf16*)w, p->C, p->n_tok, p->C, p->C, ep, s);
}

// out[M][N] = epilogue(A[M][K] B[N][K]^T): mode 0 (+ bias, + optional residual rows),
// 2 (GELU of the biased product, the biased product itself to out2) or 3 (product times
// GELU'(aux)). All row-major with pitch N.
hipError_t launch_rows_gemm_bf16(const bf16* A, int64_t lda, const bf16* B, int64_t ldb, int64_t M, int N, int K,
                                 const bf16* bias, int mode, bf16* out, bf16* out2, const bf16* aux, const bf16* res,
                                 const float* res_f32, float* out_f32, hipStream_t s) {
  EpiParams ep{};
  ep.mode = mode;
  ep.out = out;
  ep.out_f32 = out_f32;
  ep.out2 = out2;
  ep.aux = aux;
  ep.res = res;
  ep.res_f32 = res_f32;
  ep.ldc = N;
  ep.bias = bias;
  ep.qscale = 1.f;
  ep.C = N;
  return gemm_nt(A, lda, nullptr, B, ldb, M, N, K, ep, s);
}

hipError_t launch_wgrad_bf16(const bf16* A, int64_t lda, const bf16* B, int64_t ldb, int64_t T, int M, int N,
                             int splits, int64_t chunk, float* part, float* dw, float* db, hipStream_t s) {
  float* dbpart = db ? part + (int64_t)splits * M * N : nullptr;
  const int64_t tiles = (int64_t)((M + tn::BM - 1) / tn::BM) * ((N + tn::BN - 1) / tn::BN) * splits;
  k_gemm_tn<<<xcd_grid(tiles), tn::NT, 0, s>>>(A, lda, B, ldb, T, M, N, chunk, splits, part, dbpart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t threads = (int64_t)M * N / 4 + (db ? M / 4 : 0);
  k_reduce_splits<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(part, splits, M, N, dw, dbpart, db);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const void* in, void* out, int R, int Cn, hipStream_t s) {
  dim3 grid((unsigned)((Cn + 31) / 32), (unsigned)((R + 31) / 32));
  k_transpose_bf16<<<grid, 256, 0, s>>>((const bf16*)in, (bf16*)out, R, Cn);
  return hipGetLastError();
}

}  // namespace swin
