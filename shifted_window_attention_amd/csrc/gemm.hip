// bf16 MFMA GEMMs of the attention module (fp32 accumulation).
//
//   k_gemm_nt:   C[m, n] = sum_k A[m, k] * B[n, k]   (both operands K-contiguous)
//                A rows may be gathered through a row map (the cyclic shift + window
//                partition fused into the operand load), and the epilogue either
//                writes head-split q/k/v planes or scatters rows back to the grid
//                (window reverse + un-shift fused into the store).
//   k_gemm_tn:   P[s, m, n] = sum_{t in chunk s} A[t, m] * B[t, n]   (contraction over
//                tokens for the weight gradients; deterministic split-K partials)
//   k_reduce_splits: fixed-order sum of the split-K partials.
//
// Tiling for gfx950: 256 threads (4 waves of 64), v_mfma_f32_32x32x16_bf16, 64-deep
// K steps staged through LDS with 16-byte rows padded by 16 bytes so that both the
// row-wise 16-byte stores and the MFMA fragment reads are bank-conflict free.
#include "device_common.h"
#include "swin_internal.h"

namespace swin {

struct EpiParams {
  int mode;                  // 0: rows (optionally scattered), 1: head-split planes [P][nh][n_tok][hd]
  bf16* out;
  const int32_t* out_rows;   // mode 0: destination row of each C row (NULL: identity)
  int64_t ldc;               // mode 0: row pitch of out (elements)
  const bf16* bias;          // [N] or NULL
  float qscale;              // mode 1: factor for columns < C (the q block)
  int C, nh, hd;
  int64_t n_tok;
  const bf16* dot_o;         // mode 1, one plane: if set, also write dot_out[head][m] =
  float* dot_out;            //   sum over the head's columns of C[m, :] * dot_o[m, :]
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

template <int BM, int BN>
__global__ __launch_bounds__(256, 2) void k_gemm_nt(const bf16* __restrict__ A, int64_t lda,
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
  constexpr int CH_PER_ROW = BN / 8;
  static_assert((BM * CH_PER_ROW) % Cfg::NT == 0, "uniform copy-out loop");
#pragma unroll 4
  for (int c = tid; c < BM * CH_PER_ROW; c += Cfg::NT) {
    const int row = c / CH_PER_ROW;
    const int cc = (c % CH_PER_ROW) * 8;
    const int64_t m = m0 + row;
    const int n = n0 + cc;
    const bool valid = m < M && n < N;
    const bf16x8 v = *(const bf16x8*)(Cs + row * Cfg::CPITCH + cc);
    float dot = 0.f;
    if (valid) {
      bf16* dst;
      if (ep.mode == 1) {
        const int plane = n / ep.C;
        const int rem = n - plane * ep.C;
        const int head = rem / ep.hd;
        const int d = rem - head * ep.hd;
        dst = ep.out + (((int64_t)plane * ep.nh + head) * ep.n_tok + m) * ep.hd + d;
      } else {
        const int64_t orow = ep.out_rows ? (int64_t)ep.out_rows[m] : m;
        dst = ep.out + orow * ep.ldc + n;
      }
      *(bf16x8*)dst = v;
      if (ep.dot_o) {
        const bf16x8 ov = *(const bf16x8*)(ep.dot_o + m * ep.C + n);
#pragma unroll
        for (int e = 0; e < 8; ++e) dot += to_f32(v[e]) * to_f32(ov[e]);
      }
    }
    if (ep.dot_o) {
      // the 4 chunks of one (row, head) sit in 4 consecutive lanes (head_dim 32)
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
      if (valid && (c & 3) == 0) ep.dot_out[(int64_t)(n / ep.hd) * ep.n_tok + m] = dot;
    }
  }
}

// ---------------------------------------------------------------------------
// Weight-gradient GEMM: P[s][m][n] = sum over tokens t of chunk s of A[t][m] * B[t][n].
// Both operands are token-major and are staged in LDS as loaded (token rows, 16-byte
// coalesced pieces). The MFMA fragments need 8 consecutive tokens per lane at a fixed
// column; gfx950's transposing LDS read (ds_read_b64_tr_b16) returns exactly that from
// the row-major tile, so no transposed copy is made. Workgroups of the first column
// tile also produce the column sums of A (the bias gradients) for their chunk.
// ---------------------------------------------------------------------------
struct TnCfg {
  static constexpr int NT = 256;
  static constexpr int BM = 128, BN = 128, BK = 64;   // BK tokens per step
  static constexpr int PITCH = 128 + 16;               // 72 dwords: the 4 rows of a transposed read hit distinct banks
  static constexpr int TM = 2, TN = 2;                 // 4 waves, 2x2, wave tile 64x64
  static constexpr int CH = BK * (BM / 8) / NT;        // 16-byte chunks per thread and operand (4)
};

// Four bf16 from a row-major LDS tile, transposed across each 16-lane group: lane i of the
// group receives element (i % 4) of the 8-byte pieces addressed by lanes 4r + i/4, r = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// MFMA 32x32x16 fragment (8 consecutive k for column `col0 + lane%32`) from a [k][col] tile.
__device__ __forceinline__ bf16x8 frag_tr(const bf16* tile, int pitch, int k0, int col0, int lane) {
  const int g = lane >> 4, L = lane & 15;
  const bf16* base = tile + (k0 + 8 * (g >> 1) + (L >> 2)) * pitch + col0 + 16 * (g & 1) + 4 * (L & 3);
  const bf16x4 lo = lds_read_tr4(base);
  const bf16x4 hi = lds_read_tr4(base + 4 * pitch);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__global__ __launch_bounds__(256, 2) void k_gemm_tn(const bf16* __restrict__ A, int64_t lda,
                                                    const int32_t* __restrict__ a_rows,
                                                    const bf16* __restrict__ B, int64_t ldb,
                                                    const int32_t* __restrict__ b_rows, int64_t T, int M, int N,
                                                    int64_t chunk, int n_splits, float* __restrict__ part,
                                                    float* __restrict__ dbpart) {
  using Cfg = TnCfg;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * Cfg::BK * Cfg::PITCH];
  __shared__ float colsum[16][Cfg::BM];
  bf16* As = smem;                          // [BK tokens][PITCH]
  bf16* Bs = smem + Cfg::BK * Cfg::PITCH;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // tile order: N tile fastest, then M tile, then split (XCD-aware, see xcd_tile)
  const int n_nt = (N + Cfg::BN - 1) / Cfg::BN, n_mt = (M + Cfg::BM - 1) / Cfg::BM;
  int64_t ms;
  int ntile;
  if (!xcd_tile((int64_t)n_mt * n_nt * n_splits, n_nt, ms, ntile)) return;
  const int m0 = (int)(ms % n_mt) * Cfg::BM, n0 = ntile * Cfg::BN;
  const int s = (int)(ms / n_mt);
  const int64_t t_begin = (int64_t)s * chunk;
  const int64_t t_end = t_begin + chunk < T ? t_begin + chunk : T;
  const bool do_db = dbpart != nullptr && ntile == 0;

  const int crow = tid >> 4;                // token row of chunk i: crow + 16 i
  const int ccol = (tid & 15) * 8;          // column offset inside the tile
  const bool a_ok = m0 + ccol < M, b_ok = n0 + ccol < N;

  f32x16 acc[Cfg::TM][Cfg::TN];
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) acc[i][j] = f32x16{};
  float csum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) csum[e] = 0.f;

  bf16x8 ra[Cfg::CH], rb[Cfg::CH];
  auto load = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < Cfg::CH; ++i) {
      const int64_t t = t0 + crow + 16 * i;
      const bool tv = t < t_end;
      const int64_t ga = tv ? (a_rows ? (int64_t)a_rows[t] : t) : 0;
      const int64_t gb = tv ? (b_rows ? (int64_t)b_rows[t] : t) : 0;
      ra[i] = (tv && a_ok) ? *(const bf16x8*)(A + ga * lda + m0 + ccol) : bf16x8{};
      rb[i] = (tv && b_ok) ? *(const bf16x8*)(B + gb * ldb + n0 + ccol) : bf16x8{};
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < Cfg::CH; ++i) {
      *(bf16x8*)(As + (crow + 16 * i) * Cfg::PITCH + ccol) = ra[i];
      *(bf16x8*)(Bs + (crow + 16 * i) * Cfg::PITCH + ccol) = rb[i];
      if (do_db) {
#pragma unroll
        for (int e = 0; e < 8; ++e) csum[e] += to_f32(ra[i][e]);
      }
    }
  };

  if (t_begin < t_end) {
    load(t_begin);
    store();
    __syncthreads();
    for (int64_t t0 = t_begin; t0 < t_end; t0 += Cfg::BK) {
      const bool more = t0 + Cfg::BK < t_end;
      if (more) load(t0 + Cfg::BK);
#pragma unroll
      for (int ks = 0; ks < Cfg::BK / 16; ++ks) {
        bf16x8 fa[Cfg::TM], fb[Cfg::TN];
#pragma unroll
        for (int i = 0; i < Cfg::TM; ++i) fa[i] = frag_tr(As, Cfg::PITCH, ks * 16, wm * 64 + 32 * i, lane);
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j) fb[j] = frag_tr(Bs, Cfg::PITCH, ks * 16, wn * 64 + 32 * j, lane);
#pragma unroll
        for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
          for (int j = 0; j < Cfg::TN; ++j) acc[i][j] = mfma32(fa[i], fb[j], acc[i][j]);
      }
      __syncthreads();
      if (more) {
        store();
        __syncthreads();
      }
    }
  }

  float* P = part + (int64_t)s * M * N;
  const int fr = lane & 31;
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) {
      const int n = n0 + wn * 64 + 32 * j + fr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M && n < N) P[(int64_t)m * N + n] = acc[i][j][r];
      }
    }
  if (do_db) {
    // each column's 16 partial sums (one per token-row group) are combined in a fixed order
#pragma unroll
    for (int e = 0; e < 8; ++e) colsum[crow][ccol + e] = csum[e];
    __syncthreads();
    if (tid < Cfg::BM) {
      float v = 0.f;
      for (int q = 0; q < 16; ++q) v += colsum[q][tid];
      if (m0 + tid < M) dbpart[(int64_t)s * M + m0 + tid] = v;
    }
  }
}

// out[i] = sum_{s < S} part[s * stride + i], in order of s.
__global__ void k_reduce_splits(const float* __restrict__ part, int S, int64_t stride, int64_t n,
                                float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float acc = 0.f;
  for (int s = 0; s < S; ++s) acc += part[(int64_t)s * stride + i];
  out[i] = acc;
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
  constexpr int BM = 256, BN = 128;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  k_gemm_nt<BM, BN><<<xcd_grid(tiles), 256, 0, s>>>(A, lda, a_rows, B, ldb, M, N, K, ep);
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
  return gemm_nt((const bf16*)x, p->C, p->dev.perm, (const bf16*)w, p->C, p->n_tok, 3 * p->C, p->C, ep, s);
}

hipError_t launch_proj_fwd_bf16(const swin_attn_plan* p, const void* o, const void* w, const void* b, void* y,
                                hipStream_t s) {
  EpiParams ep{};
  ep.mode = 0;
  ep.out = (bf16*)y;
  ep.out_rows = p->dev.perm;  // window reverse + un-shift: slot t goes back to grid row perm[t]
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
  ep.mode = 1;  // head-split, one plane, plus D = rowsum(dO * O) per head
  ep.out = (bf16*)dO;
  ep.dot_o = (const bf16*)o;
  ep.dot_out = dd;
  ep.qscale = 1.f;
  ep.C = p->C;
  ep.nh = p->nh;
  ep.hd = p->hd;
  ep.n_tok = p->n_tok;
  return gemm_nt((const bf16*)dy, p->C, p->dev.perm, (const bf16*)wprojT, p->C, p->n_tok, p->C, p->C, ep, s);
}

hipError_t launch_dgrad_qkv_bf16(const swin_attn_plan* p, const void* dqkv, const void* wqkvT, void* dx,
                                 hipStream_t s) {
  EpiParams ep{};
  ep.mode = 0;
  ep.out = (bf16*)dx;
  ep.out_rows = p->dev.perm;
  ep.ldc = p->C;
  ep.qscale = 1.f;
  ep.C = p->C;
  return gemm_nt((const bf16*)dqkv, 3 * p->C, nullptr, (const bf16*)wqkvT, 3 * p->C, p->n_tok, p->C, 3 * p->C, ep,
                 s);
}

hipError_t launch_wgrad_bf16(const bf16* A, int64_t lda, const int32_t* a_rows, const bf16* B, int64_t ldb,
                             const int32_t* b_rows, int64_t T, int M, int N, int splits, int64_t chunk, float* part,
                             float* dw, float* db, hipStream_t s) {
  float* dbpart = db ? part + (int64_t)splits * M * N : nullptr;
  const int64_t tiles = (int64_t)((M + 127) / 128) * ((N + 127) / 128) * splits;
  k_gemm_tn<<<xcd_grid(tiles), 256, 0, s>>>(A, lda, a_rows, B, ldb, b_rows, T, M, N, chunk, splits, part, dbpart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)M * N;
  k_reduce_splits<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(part, splits, n, n, dw);
  e = hipGetLastError();
  if (e != hipSuccess || !db) return e;
  k_reduce_splits<<<(unsigned)((M + 255) / 256), 256, 0, s>>>(dbpart, splits, M, M, db);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const void* in, void* out, int R, int Cn, hipStream_t s) {
  dim3 grid((unsigned)((Cn + 31) / 32), (unsigned)((R + 31) / 32));
  k_transpose_bf16<<<grid, 256, 0, s>>>((const bf16*)in, (bf16*)out, R, Cn);
  return hipGetLastError();
}

}  // namespace swin
