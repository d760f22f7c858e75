// Fused window attention forward (bf16 MFMA, fp32 softmax), head_dim 32.
//
// For one head h and one window (TERRA section IV-A / Fig. 4: W-MSA and SW-MSA; BEAST
// "Domain-Tensor Parallelism": attention is independent per head):
//   S2 = q' k^T + log2(e) * (T[h, bin] or -inf where wrap labels differ)
//   P  = exp2(S2 - rowmax) / rowsum,  o = P v,  lse2 = rowmax + log2(rowsum)
// where q' = tau * log2(e) * q was folded into the QKV projection, so S2 = log2(e) * S.
//
// Work decomposition: one workgroup per (chunk of windows of one class, head); one wave
// per 16-query tile. Every window of a class has the same extent and label split, so a
// lane's bias + mask values (its query against every key) are computed once per
// workgroup and then serve as the initial accumulator of the Q K^T MFMA for every window
// of the chunk. A window's Q, K and V (n x 32 bf16 each) and grid rows are staged in LDS
// by direct global->LDS copies into one of two or three buffers (as many as LDS allows with
// two workgroups per CU), one or two windows ahead of the one being computed, with one
// barrier per window.
//
// The logits are computed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16), so a lane
// holds one query and 4 consecutive keys of every 16-key tile. The row max is an
// in-register reduction plus two cross-lane steps, needed only when exp2 of the raw logits
// leaves the safe range (below); the row sum comes from the matrix core
// (an all-ones operand against the same bf16 P as the PV product); and the probabilities
// of two adjacent key tiles are already the B operand of O^T = V^T P^T. The V^T operand is
// read from the row-major V tile with gfx950's transposing LDS read. A window has at most
// 256 tokens, so a query's whole key row lives in registers and the softmax is exact in a
// single pass (no online rescaling).
#include <type_traits>

#include "device_common.h"
#include "swin_internal.h"

namespace swin {

struct AttnArgs {
  const bf16* qkv;          // [3][nh][n_tok][32]
  const float* table;       // [nh][nbins]
  bf16* o;                  // [n_tok][C], grid order (row perm[slot])
  const int32_t* perm;      // window-major slot -> grid row
  float* lse;               // [nh][n_tok]
  const WorkItem* work;
  const ClassInfo* classes;
  const int32_t* class_win;
  const int32_t* win_off;
  int64_t n_tok;
  int nh, C, nbins;
  int win[3];               // nominal window (wd, wh, ww)
};

template <int NKT>
struct FwdBuf {
  static constexpr int ROWS = (NKT + 1) / 2 * 32;  // key/value rows (32-key chunks of the PV product)
  unsigned char k[ROWS * 64], v[ROWS * 64];
  unsigned char q[16 * NKT * 64];                  // wave qt's 16 query rows at 1024 qt
  int grow[NKT * 64];                              // wave qt's query grid rows at 64 qt
};

// All of the kernel's LDS is one object: the compiler then leaves the ordering of the
// direct-to-LDS copies against LDS reads to the explicit waits below.
template <int NKT>
struct FwdSmem {
  static constexpr int B = sizeof(FwdBuf<NKT>), T = 4 * (kMaxBins + kFwdMaxChunk + 16 * NKT);
  // several workgroups per CU when registers and LDS allow it (four up to 4 query tiles, three
  // up to 6, two up to 8, with the bias in fp32), with as many buffers as then fit; otherwise
  // three buffers if one workgroup fits them
  static constexpr int MIN_BLOCKS = NKT <= 4 ? 4 : (NKT <= 6 ? 3 : (NKT <= 8 ? 2 : 1));
  // the launch bound counts waves per SIMD: MIN_BLOCKS workgroups of NKT waves over the four SIMDs
  static constexpr int WAVES_PER_SIMD = (MIN_BLOCKS * NKT + 3) / 4;
  static constexpr int LDS_CAP = 160 * 1024 / MIN_BLOCKS;
  static constexpr int NBUF = 3 * B + T <= LDS_CAP ? 3 : (2 * B + T <= LDS_CAP ? 2 : (3 * B + T <= 160 * 1024 ? 3 : 2));
  FwdBuf<NKT> buf[NBUF];
  float tab[kMaxBins];  // the head's bias table times log2(e)
  int offs[kFwdMaxChunk];
  int codes[16 * NKT];  // per-token local-offset codes and wrap labels
};

template <int NKT>
__global__ __launch_bounds__(64 * NKT, FwdSmem<NKT>::WAVES_PER_SIMD) void k_attn_fwd(AttnArgs a) {
  constexpr int NKC = (NKT + 1) / 2;   // 32-key chunks of the PV product
  constexpr int ROWS = FwdBuf<NKT>::ROWS;
  constexpr int NBUF = FwdSmem<NKT>::NBUF;
  // NBUF buffers, filled by direct global->LDS copies NBUF-1 windows ahead of the one being
  // computed. A wave waits only for its own copies into the buffer it is about to read (an
  // explicit vector-memory count), then meets the other waves at a barrier that leaves that
  // count alone.
  __shared__ __attribute__((aligned(1024))) FwdSmem<NKT> sm;

  const int lane = threadIdx.x & 63;
  const int qt = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, li = lane & 15;
  const WorkItem wk = a.work[blockIdx.x];
  const int h = blockIdx.y;
  const ClassInfo ci = a.classes[wk.cls];
  const int n = ci.n;
  const int q = qt * 16 + li;
  const bool qv = q < n;
  const float* tab = a.table + (int64_t)h * a.nbins;
  for (int i = threadIdx.x; i < a.nbins; i += 64 * NKT) sm.tab[i] = tab[i] * kLog2e;
  for (int i = threadIdx.x; i < wk.count; i += 64 * NKT) sm.offs[i] = a.win_off[a.class_win[wk.first + i]];
  if (threadIdx.x < 16 * NKT)
    sm.codes[threadIdx.x] = threadIdx.x < n ? token_code(threadIdx.x, ci.ext, ci.split, a.win) : 0;
  // V rows past the copied 16 NKT (odd tile count) feed the last PV chunk: keep them zero
  if constexpr (ROWS > 16 * NKT) {
    constexpr int TAIL = (ROWS - 16 * NKT) * 64 / 4;
    for (int i = threadIdx.x; i < TAIL * NBUF; i += 64 * NKT)
      ((int*)(sm.buf[i / TAIL].v + 16 * NKT * 64))[i % TAIL] = 0;
  }
  __syncthreads();  // table, offsets, codes and zero rows in LDS

  const bf16* Qh = a.qkv + ((int64_t)(0 * a.nh + h) * a.n_tok) * 32;
  const bf16* Kh = a.qkv + ((int64_t)(1 * a.nh + h) * a.n_tok) * 32;
  const bf16* Vh = a.qkv + ((int64_t)(2 * a.nh + h) * a.n_tok) * 32;
  // Copies of rows past n read row n-1 instead: those keys are masked (-inf logits, zero
  // probabilities) and those queries' outputs are dropped, so any finite values will do.
  // Each wave issues exactly four copies per window: the 16-row slabs qt of K, V and Q and
  // the grid rows of its 16 queries (lanes 16..63 repeat them).
  constexpr int COPIES = 4;
  const int crow = 16 * qt + (lane >> 2);
  const int cchunk = (lane & 3) ^ swz(crow);
  const int crow_src = crow < n ? crow : n - 1;
  const int grow_src = 16 * qt + li < n ? 16 * qt + li : n - 1;
  auto stage = [&](int w) {
    FwdBuf<NKT>& b = sm.buf[w % NBUF];
    const int64_t off = sm.offs[w];
    const int64_t src = (off + crow_src) * 32 + 8 * cchunk;
    lds_copy16(Kh + src, b.k + 1024 * qt);
    lds_copy16(Vh + src, b.v + 1024 * qt);
    lds_copy16(Qh + src, b.q + 1024 * qt);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(a.perm + off + grow_src),
                                     (__attribute__((address_space(3))) void*)(b.grow + 64 * qt), 4, 0, 0);
  };
  for (int w = 0; w < NBUF - 1 && w < wk.count; ++w) stage(w);

  // bias + mask of this lane's query against every key; keys past n are masked, and
  // queries past n (whose outputs are dropped) get finite zeros. The values are rounded to
  // fp16 (|error| <= 2^-11 |bias|, -inf exact) as in the backward, which recomputes P from the
  // saved LSE with the same rounded logits. Held in fp32 up to 10 query tiles (an fp16 copy
  // would cost a conversion per pair and window); beyond that as fp16, which leaves registers
  // for the logits.
  typedef typename std::conditional<NKT <= 10, float, _Float16>::type bias_t;
  typedef bias_t h4 __attribute__((ext_vector_type(4)));
  const int code0 = code0_of(a.win);
  const int cq = sm.codes[q];
  h4 bias[NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    const int4 ck = *(const int4*)(sm.codes + 16 * kt + 4 * g);
    const int kk[4] = {ck.x, ck.y, ck.z, ck.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = 16 * kt + 4 * g + i;
      bias[kt][i] = (bias_t)(_Float16)(!qv ? 0.f : (k >= n ? -INFINITY : pair_bias_codes(cq, kk[i], code0, sm.tab)));
    }
  }

  // a window's results are stored in the next window, before that window's copies are issued
  bf16x4 ov[2] = {};
  float lse_v = 0.f;
  int64_t prev_off = -1;
  int prev_row = 0;  // grid row of this lane's query in the previous window
  // fragment offsets inside a tile: row 16 t + li of slab t, and the transposed V^T reads
  // (rows 32 c + 4 g + li/4 and +16, columns 4 (li % 4) and +16) are these lane offsets plus
  // constants, because rows that differ by a multiple of 16 have the same swizzle
  const int kq_off = li * 64 + 16 * (g ^ swz(li));
  const int vr = 4 * g + (li >> 2);
  const int vt_off0 = swz_off(vr, 4 * (li & 3)), vt_off1 = swz_off(vr, 16 + 4 * (li & 3));
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = to_bf16(1.f);
  for (int w = 0; w < wk.count; ++w) {
    const FwdBuf<NKT>& cur = sm.buf[w % NBUF];
    // Issue order: the first NBUF-1 windows' copies, then per window w: the stores of window
    // w-1, then the copies of window w+NBUF-1. Operations complete in issue order, so the
    // copies of window w are done once at most the copies of windows w+1 .. w+NBUF-2 are
    // outstanding (stores issued in between only make that wait stricter).
    {
      const int later = wk.count - 1 - w < NBUF - 2 ? wk.count - 1 - w : NBUF - 2;  // windows staged after w
      vm_wait(COPIES * later);
    }
    // every wave's copies into `cur` have landed, and every wave is done with window w-1
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (prev_off >= 0) {
      const bf16x8 o8 = pair_cols(ov[0], ov[1], g);
      if (qv) {
        *(bf16x8*)(a.o + (int64_t)prev_row * a.C + h * 32 + pair_col(g)) = o8;
        if (g == 0) a.lse[(int64_t)h * a.n_tok + prev_off + q] = lse_v;
      }
    }
    if (w + NBUF - 1 < wk.count) stage(w + NBUF - 1);  // into the buffer window w-1 used
    const bf16x8 bq = *(const bf16x8*)(cur.q + kq_off + 1024 * qt);
    f32x4 s[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) asm volatile("" : "+v"(bias[kt]));  // expand per window, not hoisted
    f32x4 oacc[2], lacc;
    float m;
    if constexpr (NKT <= 10) {
      auto logits = [&]() {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          const f32x4 b4 = {(float)bias[kt][0], (float)bias[kt][1], (float)bias[kt][2], (float)bias[kt][3]};
          s[kt] = mfma16(*(const bf16x8*)(cur.k + kq_off + 1024 * kt), bq, b4);
        }
      };
      // O^T = V^T P^T, and the row sums of the same bf16 P from an all-ones A operand: every row
      // of that product is the lane's query sum, so no cross-lane reduction is needed
      auto pv = [&]() {
        oacc[0] = oacc[1] = lacc = f32x4{};
#pragma unroll
        for (int c = 0; c < NKC; ++c) {
          bf16x8 pb;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pb[i] = to_bf16(s[2 * c][i]);
            pb[4 + i] = (2 * c + 1 < NKT) ? to_bf16(s[2 * c + 1][i]) : to_bf16(0.f);
          }
          bf16x8 v0, v1;
          tile_frag_tr2_at(cur.v + 2048 * c, vt_off0, vt_off1, v0, v1);
          oacc[0] = mfma16(v0, pb, oacc[0]);
          oacc[1] = mfma16(v1, pb, oacc[1]);
          lacc = mfma16(ones, pb, lacc);
        }
      };
      // The softmax is invariant to a per-row offset, so the exponent offset is needed only to
      // keep exp2 in range, and the first pass takes none: P = exp2(S2), l = rowsum(P). A row sum
      // in [2^-60, 2^100] means no term overflowed and every term that underflowed lies below
      // 2^-58 of the row's largest; otherwise (also for inf or NaN sums) the wave recomputes its
      // logits and takes the row maximum m as the offset. Either way lse2 = offset + log2(l).
      logits();
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[kt][i] = fast_exp2(s[kt][i]);
      pv();
      m = 0.f;
      if (__builtin_amdgcn_ballot_w64(!(lacc[0] >= 0x1p-60f && lacc[0] <= 0x1p100f)) != 0) {
        logits();
        m = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = fmaxf(m, s[kt][i]);
        m = wave_max_xor16_32(m);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[kt][i] = fast_exp2(s[kt][i] - m);
        pv();
      }
    } else {
      // beyond 10 key tiles the two passes' live ranges would spill: always the offset m
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const f32x4 b4 = {(float)bias[kt][0], (float)bias[kt][1], (float)bias[kt][2], (float)bias[kt][3]};
        s[kt] = mfma16(*(const bf16x8*)(cur.k + kq_off + 1024 * kt), bq, b4);
      }
      m = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, s[kt][i]);
      m = wave_max_xor16_32(m);
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[kt][i] = fast_exp2(s[kt][i] - m);
      oacc[0] = oacc[1] = lacc = f32x4{};
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[i] = to_bf16(s[2 * c][i]);
          pb[4 + i] = (2 * c + 1 < NKT) ? to_bf16(s[2 * c + 1][i]) : to_bf16(0.f);
        }
        bf16x8 v0, v1;
        tile_frag_tr2_at(cur.v + 2048 * c, vt_off0, vt_off1, v0, v1);
        oacc[0] = mfma16(v0, pb, oacc[0]);
        oacc[1] = mfma16(v1, pb, oacc[1]);
        lacc = mfma16(ones, pb, lacc);
      }
    }
    const float l = lacc[0];
    const float inv = __builtin_amdgcn_rcpf(l);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[dt][i] = to_bf16(oacc[dt][i] * inv);
    lse_v = m + fast_log2(l);
    prev_off = sm.offs[w];
    prev_row = cur.grow[64 * qt + li];
  }
  if (prev_off >= 0) {
    const bf16x8 o8 = pair_cols(ov[0], ov[1], g);
    if (qv) {
      *(bf16x8*)(a.o + (int64_t)prev_row * a.C + h * 32 + pair_col(g)) = o8;
      if (g == 0) a.lse[(int64_t)h * a.n_tok + prev_off + q] = lse_v;
    }
  }
}

template <int NKT>
static void launch_one(const AttnArgs& a, int n_items, int nh, hipStream_t s) {
  k_attn_fwd<NKT><<<dim3((unsigned)n_items, (unsigned)nh), 64 * NKT, 0, s>>>(a);
}

typedef void (*fwd_launcher)(const AttnArgs&, int, int, hipStream_t);
static const fwd_launcher kFwd[17] = {nullptr,          launch_one<1>,  launch_one<2>,  launch_one<3>,
                                      launch_one<4>,    launch_one<5>,  launch_one<6>,  launch_one<7>,
                                      launch_one<8>,    launch_one<9>,  launch_one<10>, launch_one<11>,
                                      launch_one<12>,   launch_one<13>, launch_one<14>, launch_one<15>,
                                      launch_one<16>};

// Workgroups of the k_attn_fwd<nqt> launch that one CU holds at once (at least 1).
int attn_fwd_blocks_per_cu(int nqt) {
  static const void* const kern[17] = {
      nullptr,
      (const void*)k_attn_fwd<1>,  (const void*)k_attn_fwd<2>,  (const void*)k_attn_fwd<3>,  (const void*)k_attn_fwd<4>,
      (const void*)k_attn_fwd<5>,  (const void*)k_attn_fwd<6>,  (const void*)k_attn_fwd<7>,  (const void*)k_attn_fwd<8>,
      (const void*)k_attn_fwd<9>,  (const void*)k_attn_fwd<10>, (const void*)k_attn_fwd<11>, (const void*)k_attn_fwd<12>,
      (const void*)k_attn_fwd<13>, (const void*)k_attn_fwd<14>, (const void*)k_attn_fwd<15>, (const void*)k_attn_fwd<16>};
  int n = 0;
  if (nqt < 1 || nqt > 16 || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern[nqt], 64 * nqt, 0) != hipSuccess)
    n = 1;
  return n < 1 ? 1 : n;
}

hipError_t launch_attn_fwd_bf16(const swin_attn_plan* p, const void* qkv, const float* table, void* o, float* lse,
                                hipStream_t s) {
  if (p->tiled) return launch_tiled_fwd_bf16(p, qkv, table, o, lse, s);
  AttnArgs a{};
  a.qkv = (const bf16*)qkv;
  a.table = table;
  a.o = (bf16*)o;
  a.perm = p->dev.perm;
  a.lse = lse;
  a.classes = p->dev.classes;
  a.class_win = p->dev.class_win;
  a.win_off = p->dev.win_off;
  a.n_tok = p->n_tok;
  a.nh = p->nh;
  a.C = p->C;
  a.nbins = p->nbins;
  for (int i = 0; i < 3; ++i) a.win[i] = p->d.window[i];
  for (const auto& r : p->fwd_ranges) {
    a.work = p->dev.fwd_work + r.begin;
    kFwd[r.nqt](a, r.count, p->nh, s);
  }
  return hipGetLastError();
}

}  // namespace swin
