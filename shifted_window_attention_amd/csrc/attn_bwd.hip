// Window attention backward (bf16 MFMA, fp32 softmax gradients), head_dim 32.
//
// With S2 = log2(e) S, P = exp2(S2 - lse2), natural-unit gradients:
//   dV = P^T dO;  dP = dO V^T;  D = rowsum(dO * O);  dS = P * (dP - D);
//   dq = tau dS K;  dk = tau dS^T q = (dS^T q') / log2(e);  dT[h, bin] += dS
// (q' = tau log2(e) q is the stored query). The inverse routes carry these gradients
// back to their sources (TERRA section IV-D).
//
// D = rowsum(dO * O) comes (negated) from the epilogue of the GEMM that produces dO; the
// logit and dP products start from bias - lse and -D, which saves two subtractions per pair.
//
// Work decomposition: one workgroup per (chunk of windows of one class, head), one wave
// per 16-key tile. Each window's Q', dO, K, V, lse and D are staged in LDS by direct
// global->LDS copies, double-buffered so window w+1 is copied while window w is computed. A lane holds one key and 4 consecutive queries of every 16-query tile
// (S = Q K^T on v_mfma_f32_16x16x32_bf16), so dV^T = dO^T P and dK^T = Q'^T dS contract
// over queries inside the wave: P and dS of two adjacent query tiles are directly the B
// operand, and dO^T, Q'^T come from the row-major LDS tiles through gfx950's transposing
// LDS read. dQ contracts over keys, i.e. over waves: dS goes through LDS once (bf16) and
// every wave then forms dQ^T = K^T dS^T for one query tile.
//
// Bias gradient without global atomics: all windows of a chunk share one class, so a
// lane's (query, key) positions are the same in every window and its dS values (as rounded
// to bf16 for the dK and dQ products) are summed over the chunk in fp32 registers, on the
// matrix core against a 0/1 selector operand. Once per workgroup the per-position sums are binned into
// the relative-position table in LDS, each bin owned by one thread and filled in a fixed
// order, and the workgroup writes one partial table. A second kernel adds the partials
// in order of work item. Every reduction therefore has a fixed order and repeated calls
// are bitwise identical.
#include "device_common.h"
#include "swin_internal.h"

namespace swin {

struct BwdArgs {
  const bf16* qkv;          // saved [3][nh][n_tok][32] (q pre-scaled)
  const bf16* o;            // saved [n_tok][C], grid order
  const float* lse;         // saved [nh][n_tok] (log2 units)
  const bf16* dO;           // [nh][n_tok][32]
  const float* dd;          // [nh][n_tok]: -D = -rowsum(dO * O)
  const float* table;       // [nh][nbins]
  bf16* dqkv;               // [n_tok][3C], grid order (row perm[slot])
  const int32_t* perm;      // window-major slot -> grid row
  float* dbias_part;        // [n_items_total][nh][nbins]
  const WorkItem* work;     // this launch's items
  int item_base;            // index of work[0] among all backward work items
  const ClassInfo* classes;
  const int32_t* class_win;
  const int32_t* win_off;
  int64_t n_tok;
  int nh, C, nbins;
  int win[3];
  float tau;
};

template <int NKT>
struct BwdBuf {
  static constexpr int ROWS = (NKT + 1) / 2 * 32;  // staged rows per tile (32-row chunks)
  static constexpr int FROWS = (ROWS + 63) / 64 * 64;  // float rows: whole 64-lane copies
  unsigned char q[ROWS * 64], dO[ROWS * 64], k[ROWS * 64], v[ROWS * 64];
  float lse[FROWS], dd[FROWS];
  int grow[FROWS];  // grid row of each token of the window
};

template <int NKT>
__global__ __launch_bounds__(64 * NKT, 1) void k_attn_bwd(BwdArgs a) {
  constexpr int NKC = (NKT + 1) / 2;
  constexpr int NT = 64 * NKT;
  constexpr int ROWS = BwdBuf<NKT>::ROWS;
  // dS is kept transposed, dSt[key][query], so a lane's 4 consecutive queries of one key
  // are one 8-byte store; the pitch (an odd multiple of 8 bytes past a 16-byte multiple)
  // puts the 16 keys x 2 query groups of a half-wave store on distinct banks
  constexpr int SPT = 16 * NKT + 8;
  // Binning slab: rows of 16 NKT fp32 pair sums, laid over the two staging buffers and the dS
  // tile once the window loop is done (rows [0, RA) in bufA, [RA, 2 RA) in bufB, the rest in
  // dSt); usually all 16 NKT query rows fit, so one pass bins the whole chunk.
  // slab row pitch: 16 NKT + 4 floats, so the 4 query groups of a store land on distinct banks
  constexpr int KCOLS = 16 * NKT + 4;
  constexpr int KROW = KCOLS * 4;                                       // bytes per slab row
  constexpr int RA = (int)sizeof(BwdBuf<NKT>) / KROW;
  constexpr int RS = (int)(ROWS * (16 * NKT + 8) * sizeof(bf16)) / KROW;
  constexpr int SLAB = 2 * RA + RS;
  static_assert(RA >= 1 && SLAB >= 16, "LDS too small for the bias-gradient slab");
  static_assert(BwdBuf<NKT>::FROWS % 64 == 0 && BwdBuf<NKT>::FROWS >= ROWS, "float rows are whole copies");
  // Two staging buffers (separate objects, loop unrolled by two, see the forward kernel)
  // filled by direct global->LDS copies while the other one is computed, dS for dQ, and
  // the per-bin partial sums.
  __shared__ __attribute__((aligned(1024))) BwdBuf<NKT> bufA;
  __shared__ __attribute__((aligned(1024))) BwdBuf<NKT> bufB;
  __shared__ __attribute__((aligned(16))) bf16 dSt[ROWS * SPT];
  __shared__ int offs[kMaxChunk];
  __shared__ int codes[16 * NKT];  // per-token local-offset codes and wrap labels
  extern __shared__ float dyn_lds[];   // [2 nbins]: bias-gradient bins, then the scaled table
  float* bins_lds = dyn_lds;
  float* tab_lds = dyn_lds + a.nbins;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int kt = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, li = lane & 15;
  const WorkItem wk = a.work[blockIdx.x];
  const int h = blockIdx.y;
  const ClassInfo ci = a.classes[wk.cls];
  const int n = ci.n;
  const int key = 16 * kt + li;
  const float* tab = a.table + (int64_t)h * a.nbins;
  for (int i = tid; i < wk.count; i += NT) offs[i] = a.win_off[a.class_win[wk.first + i]];
  if (tid < 16 * NKT) codes[tid] = tid < n ? token_code(tid, ci.ext, ci.split, a.win) : 0;
  const int64_t off0 = a.win_off[a.class_win[wk.first]];

  const bf16* Qh = a.qkv + ((int64_t)(0 * a.nh + h) * a.n_tok) * 32;
  const bf16* Kh = a.qkv + ((int64_t)(1 * a.nh + h) * a.n_tok) * 32;
  const bf16* Vh = a.qkv + ((int64_t)(2 * a.nh + h) * a.n_tok) * 32;
  const bf16* dOh = a.dO + ((int64_t)h * a.n_tok) * 32;
  const float* LSEh = a.lse + (int64_t)h * a.n_tok;
  const float* Dh = a.dd + (int64_t)h * a.n_tok;
  // rows past n arrive as zeros (buffer range = the window's n rows)
  auto stage = [&](int64_t off, BwdBuf<NKT>& b) {
    const uint32_t bytes = (uint32_t)n * 64;
    stage_rows(make_rsrc(Qh + off * 32, bytes), b.q, ROWS, kt, NKT, lane);
    stage_rows(make_rsrc(dOh + off * 32, bytes), b.dO, ROWS, kt, NKT, lane);
    stage_rows(make_rsrc(Kh + off * 32, bytes), b.k, ROWS, kt, NKT, lane);
    stage_rows(make_rsrc(Vh + off * 32, bytes), b.v, ROWS, kt, NKT, lane);
    stage_floats(make_rsrc(LSEh + off, (uint32_t)n * 4), b.lse, BwdBuf<NKT>::FROWS, kt, NKT, lane);
    stage_floats(make_rsrc(Dh + off, (uint32_t)n * 4), b.dd, BwdBuf<NKT>::FROWS, kt, NKT, lane);
    stage_floats(make_rsrc(a.perm + off, (uint32_t)n * 4), (float*)b.grow, BwdBuf<NKT>::FROWS, kt, NKT, lane);
  };
  // key rows of dS that no wave owns (odd tile count) are read by dQ: keep them zero
  if constexpr (ROWS > 16 * NKT) {
    for (int c = tid; c < (ROWS - 16 * NKT) * SPT; c += NT) dSt[16 * NKT * SPT + c] = to_bf16(0.f);
  }
  for (int i = tid; i < a.nbins; i += NT) {
    bins_lds[i] = 0.f;
    tab_lds[i] = tab[i] * kLog2e;
  }
  stage(off0, bufA);
  __syncthreads();  // table, offsets and zeroed regions in LDS

  // lane's bias + mask for every query tile (S layout: key fixed, queries 16 qt + 4 g + i),
  // held as fp16 to leave registers for the dS sums: |error| <= 2^-11 |bias|, -inf exact
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  const int code0 = code0_of(a.win);
  const int ckey = codes[key];
  h4 bias[NKT];
  f32x4 dbacc[NKT];
#pragma unroll
  for (int qt = 0; qt < NKT; ++qt) {
    const int4 cq = *(const int4*)(codes + 16 * qt + 4 * g);
    const int qq[4] = {cq.x, cq.y, cq.z, cq.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 16 * qt + 4 * g + i;
      bias[qt][i] = (_Float16)((q >= n || key >= n) ? -INFINITY : pair_bias_codes(qq[i], ckey, code0, tab_lds));
      dbacc[qt][i] = 0.f;
    }
  }
  const int C = a.C;
  const float inv_log2e = 1.f / kLog2e;
  // Selector operands for the bias-gradient sums on the matrix core: sel[u] (16 x 32, A operand)
  // has a one at row r, column 8 (r / 4) + 4 u + r % 4, the slot of query 16 u + r of a chunk in
  // the dS operand, so mfma16(sel[u], dS chunk, acc) adds the chunk's tile-u dS (as rounded to
  // bf16 for the dK and dQ products) to acc in the dbacc layout.
  bf16x8 sel[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[u][e] = to_bf16((g == (li >> 2) && e == 4 * u + (li & 3)) ? 1.f : 0.f);
  __syncthreads();

  // A __syncthreads() waits for every outstanding vector memory operation, the copies of
  // the next window included: those copies land during the first half of the window (S, P,
  // dP, dK, dV), before the mid-window barrier. (An LDS-only barrier there, which keeps them
  // in flight through the dQ half, measured slower.) No store is outstanding at the
  // mid-window barrier: dK and dV are stored right after it, and dq at the start of the
  // next window, after the next copies are issued.
  bf16x4 pq[2] = {};
  int64_t prev_off = -1;
  int prev_row = 0;  // grid row of this lane's dq row in the previous window
  auto flush = [&]() {
    if (prev_off < 0) return;
    const int q = 16 * kt + li;
    const bf16x8 dq8 = pair_cols(pq[0], pq[1], g);
    if (q < n) *(bf16x8*)(a.dqkv + (int64_t)prev_row * (3 * C) + h * 32 + pair_col(g)) = dq8;
  };

  auto window = [&](int w, const BwdBuf<NKT>& cur, BwdBuf<NKT>& nxt) {
    const int64_t off = offs[w];
    if (w + 1 < wk.count) stage(offs[w + 1], nxt);  // overlaps with this window's compute
    flush();
    // keep the packed fp16 bias opaque per window so its fp32 expansion is not hoisted out
    // of the loop (that would cost the registers the packing saves)
#pragma unroll
    for (int qt = 0; qt < NKT; ++qt) asm volatile("" : "+v"(bias[qt]));
    // the wave's own key tile as B operands (K^T for S, V^T for dP)
    const bf16x8 kb = tile_frag(cur.k, key, g);
    const bf16x8 vb = tile_frag(cur.v, key, g);
    f32x4 dvacc[2] = {f32x4{}, f32x4{}}, dkacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      bf16x8 pb = {}, sb = {};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int qt = 2 * c + u;
        if (qt < NKT) {
          // the products start from bias - lse and from -D, so they end as log2(P) and dP - D
          const f32x4 l4 = *(const f32x4*)(cur.lse + 16 * qt + 4 * g);
          const f32x4 nd4 = *(const f32x4*)(cur.dd + 16 * qt + 4 * g);
          const u32x2 bp = __builtin_bit_cast(u32x2, bias[qt]);
          const f32x4 b4 = {half_lo_minus(bp[0], l4[0]), half_hi_minus(bp[0], l4[1]), half_lo_minus(bp[1], l4[2]),
                            half_hi_minus(bp[1], l4[3])};
          const f32x4 s = mfma16(tile_frag(cur.q, 16 * qt + li, g), kb, b4);
          const f32x4 dp = mfma16(tile_frag(cur.dO, 16 * qt + li, g), vb, nd4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(s[i]);
            pb[4 * u + i] = to_bf16(p);
            sb[4 * u + i] = to_bf16(p * dp[i]);
          }
          *(bf16x4*)(dSt + key * SPT + 16 * qt + 4 * g) = bf16x4{sb[4 * u], sb[4 * u + 1], sb[4 * u + 2], sb[4 * u + 3]};
        }
      }
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        dvacc[dt] = mfma16(tile_frag_tr(cur.dO, 32 * c, 16 * dt, g, li), pb, dvacc[dt]);
        dkacc[dt] = mfma16(tile_frag_tr(cur.q, 32 * c, 16 * dt, g, li), sb, dkacc[dt]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (2 * c + u < NKT) dbacc[2 * c + u] = mfma16(sel[u], sb, dbacc[2 * c + u]);
      // bound live ranges to one query chunk (the two tiles inside a chunk may interleave: the
      // second tile's S and dP products overlap the first tile's exp and conversions)
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();  // dS complete; the next window's copies have landed
    {
      bf16x4 k4[2], v4[2];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          k4[dt][i] = to_bf16(dkacc[dt][i] * inv_log2e);
          v4[dt][i] = to_bf16(dvacc[dt][i]);
        }
      const bf16x8 k8 = pair_cols(k4[0], k4[1], g), v8 = pair_cols(v4[0], v4[1], g);
      if (key < n) {
        bf16* row = a.dqkv + (int64_t)cur.grow[key] * (3 * C) + h * 32 + pair_col(g);
        *(bf16x8*)(row + C) = k8;
        *(bf16x8*)(row + 2 * C) = v8;
      }
    }
    // dQ^T for query tile kt: K^T (transposed read of K) times dS^T, whose columns (8 keys
    // at one query) come from dSt through the transposing LDS read
    {
      // lane j of each 16-lane group addresses key row 4g + j/4, queries 16 kt + 4 (j%4) ..
      const bf16* dq_src = dSt + (4 * g + (li >> 2)) * SPT + 16 * kt + 4 * (li & 3);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        f32x4 dq = f32x4{};
#pragma unroll
        for (int c = 0; c < NKC; ++c) {
          const bf16x4 lo = lds_read_tr(dq_src + 32 * c * SPT);
          const bf16x4 hi = lds_read_tr(dq_src + (32 * c + 16) * SPT);
          const bf16x8 sq = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          dq = mfma16(tile_frag_tr(cur.k, 32 * c, 16 * dt, g, li), sq, dq);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) pq[dt][i] = to_bf16(dq[i] * a.tau);
      }
    }
    prev_off = off;
    prev_row = cur.grow[16 * kt + li];
    __syncthreads();  // window w+1 staged; this buffer and dS are free
  };
  for (int w = 0; w < wk.count; w += 2) {
    window(w, bufA, bufB);
    if (w + 1 < wk.count) window(w + 1, bufB, bufA);
  }
  flush();

  // bin the chunk's per-position dS sums into the relative-position table, slab by slab
  auto slab_row = [&](int lr) -> float* {
    if (lr < RA) return (float*)&bufA + lr * KCOLS;
    if (lr < 2 * RA) return (float*)&bufB + (lr - RA) * KCOLS;
    return (float*)dSt + (lr - 2 * RA) * KCOLS;
  };
  for (int q0 = 0; q0 < 16 * NKT; q0 += SLAB) {
#pragma unroll
    for (int qt = 0; qt < NKT; ++qt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = 16 * qt + 4 * g + i;
        if (q >= q0 && q < q0 + SLAB) slab_row(q - q0)[key] = dbacc[qt][i];
      }
    __syncthreads();
    for (int b = tid; b < a.nbins; b += NT) {
      // bin b <-> offset (query minus key) along each axis; its pairs are (q, q - offset)
      const int tw = 2 * a.win[2] - 1, th = 2 * a.win[1] - 1;
      const int rw = b % tw - (a.win[2] - 1);
      const int rh = (b / tw) % th - (a.win[1] - 1);
      const int rd = b / (tw * th) - (a.win[0] - 1);
      const int dk = (rd * ci.ext[1] + rh) * ci.ext[2] + rw;  // token-index offset of the pair
      float sum = bins_lds[b];
      const int q1 = q0 + SLAB < n ? q0 + SLAB : n;
      // queries whose key (q - offset) lies inside the window extent, walked row by row
      for (int qd = rd > 0 ? rd : 0; qd < ci.ext[0] + (rd < 0 ? rd : 0); ++qd)
        for (int qh = rh > 0 ? rh : 0; qh < ci.ext[1] + (rh < 0 ? rh : 0); ++qh) {
          const int row = (qd * ci.ext[1] + qh) * ci.ext[2];
          const int w0 = rw > 0 ? rw : 0, w1 = ci.ext[2] + (rw < 0 ? rw : 0);
          for (int qw = w0; qw < w1; ++qw) {
            const int q = row + qw;
            if (q >= q0 && q < q1) sum += slab_row(q - q0)[q - dk];
          }
        }
      bins_lds[b] = sum;
    }
    __syncthreads();
  }
  float* part = a.dbias_part + ((int64_t)(a.item_base + blockIdx.x) * a.nh + h) * a.nbins;
  for (int b = tid; b < a.nbins; b += NT) part[b] = bins_lds[b];
}

// dT[h][b] = sum over work items (in order) of the partial tables.
// The partials are loaded 16 at a time before they are added (in item order), so that the
// loads of a thread overlap instead of each waiting for the previous add.
__global__ void k_dbias_reduce(const float* __restrict__ part, int n_items, int per_item, float* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= per_item) return;
  constexpr int U = 16;
  const float* src = part + i;
  float acc = 0.f;
  int it = 0;
  for (; it + U <= n_items; it += U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[(int64_t)(it + u) * per_item];
#pragma unroll
    for (int u = 0; u < U; ++u) acc += v[u];
  }
  for (; it < n_items; ++it) acc += src[(int64_t)it * per_item];
  out[i] = acc;
}

template <int NKT>
static void launch_bwd_one(const BwdArgs& a, int n_items, int nh, size_t dyn, hipStream_t s) {
  k_attn_bwd<NKT><<<dim3((unsigned)n_items, (unsigned)nh), 64 * NKT, dyn, s>>>(a);
}

// Two staging buffers of Q', dO, K, V plus dS fit the 160 KB of LDS up to 10 key tiles.
typedef void (*bwd_launcher)(const BwdArgs&, int, int, size_t, hipStream_t);
static const bwd_launcher kBwd[kMaxBwdTiles + 1] = {nullptr,           launch_bwd_one<1>, launch_bwd_one<2>,
                                                    launch_bwd_one<3>, launch_bwd_one<4>, launch_bwd_one<5>,
                                                    launch_bwd_one<6>, launch_bwd_one<7>, launch_bwd_one<8>,
                                                    launch_bwd_one<9>, launch_bwd_one<10>};

// Workgroups of the k_attn_bwd<nqt> launch (dynamic LDS of dyn bytes) that one CU holds at once.
int attn_bwd_blocks_per_cu(int nqt, size_t dyn) {
  static const void* const kern[kMaxBwdTiles + 1] = {
      nullptr,
      (const void*)k_attn_bwd<1>, (const void*)k_attn_bwd<2>, (const void*)k_attn_bwd<3>, (const void*)k_attn_bwd<4>,
      (const void*)k_attn_bwd<5>, (const void*)k_attn_bwd<6>, (const void*)k_attn_bwd<7>, (const void*)k_attn_bwd<8>,
      (const void*)k_attn_bwd<9>, (const void*)k_attn_bwd<10>};
  int n = 0;
  if (nqt < 1 || nqt > kMaxBwdTiles ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern[nqt], 64 * nqt, dyn) != hipSuccess)
    n = 1;
  return n < 1 ? 1 : n;
}

hipError_t launch_dproj_bf16(const swin_attn_plan* p, const void* dy, const void* wprojT, void* dO, const void* o,
                             float* dd, hipStream_t s);
hipError_t launch_dgrad_qkv_bf16(const swin_attn_plan* p, const void* dqkv, const void* wqkvT, void* dx,
                                 float* dx32, hipStream_t s);

hipError_t launch_bwd_bf16(const swin_attn_plan* p, const void* dy, const void* x, const void* w_qkv,
                           const void* w_proj, const float* table, const void* saved, void* dx, float* dw_qkv,
                           float* db_qkv, float* dw_proj, float* db_proj, float* dtable, void* ws,
                           hipStream_t s, float* dx32) {
  const char* sv = (const char*)saved;
  return launch_bwd_bf16_parts(p, dy, x, w_qkv, w_proj, table, sv, sv + p->saved_qkv,
                               (const float*)(sv + p->saved_qkv + p->saved_o), dx, dw_qkv, db_qkv, dw_proj, db_proj,
                               dtable, ws, s, dx32);
}

hipError_t launch_bwd_bf16_parts(const swin_attn_plan* p, const void* dy, const void* x, const void* w_qkv,
                                 const void* w_proj, const float* table, const void* qkv_v, const void* o_v,
                                 const float* lse, void* dx, float* dw_qkv, float* db_qkv, float* dw_proj,
                                 float* db_proj, float* dtable, void* ws, hipStream_t s, float* dx32) {
  const int C = p->C;
  const bf16* qkv = (const bf16*)qkv_v;
  const bf16* o = (const bf16*)o_v;
  char* w = (char*)ws;
  bf16* dO = (bf16*)w;
  bf16* dqkv = (bf16*)(w + p->bwd_do);
  bf16* wprojT = (bf16*)(w + p->bwd_do + p->bwd_dqkv);
  bf16* wqkvT = wprojT + (size_t)C * C;
  float* part = (float*)(w + p->bwd_do + p->bwd_dqkv + p->bwd_wt);
  float* dbias_part = (float*)(w + p->bwd_do + p->bwd_dqkv + p->bwd_wt + p->bwd_part);
  float* dd = (float*)(w + p->bwd_do + p->bwd_dqkv + p->bwd_wt + p->bwd_part + p->bwd_dbias_part);

  hipError_t e = trace_mark(s);
  if (e == hipSuccess) e = launch_transpose_bf16(w_proj, wprojT, C, C, s);
  if (e == hipSuccess) e = launch_transpose_bf16(w_qkv, wqkvT, 3 * C, C, s);
  if (e == hipSuccess) e = trace_mark(s);
  // proj backward: dO = gather(dy) W_proj (head-split), dW_proj = gather(dy)^T o, db_proj
  if (e == hipSuccess) e = launch_dproj_bf16(p, dy, wprojT, dO, o, dd, s);
  if (e == hipSuccess) e = trace_mark(s);
  if (e == hipSuccess)
    e = launch_wgrad_bf16((const bf16*)dy, C, o, C, p->n_tok, C, C, p->wgrad_splits_proj, p->wgrad_chunk_proj, part,
                          dw_proj, db_proj, s);
  if (e == hipSuccess) e = trace_mark(s);
  if (e != hipSuccess) return e;
  if (p->tiled_bwd) {
    // windows over 160 tokens, wider heads or large tables: the tiled kernels; dT goes through
    // a fixed-point accumulator held where the one-tile path keeps its partials
    e = launch_tiled_bwd_bf16(p, qkv, lse, dO, dd, table, dqkv, (unsigned long long*)dbias_part, dtable, s);
    if (e == hipSuccess) e = trace_mark(s);
    if (e == hipSuccess) e = trace_mark(s);
  } else {
    // attention core backward
    BwdArgs a{};
    a.qkv = qkv;
    a.o = o;
    a.lse = lse;
    a.dO = dO;
    a.dd = dd;
    a.table = table;
    a.dqkv = dqkv;
    a.perm = p->dev.perm;
    a.dbias_part = dbias_part;
    a.classes = p->dev.classes;
    a.class_win = p->dev.class_win;
    a.win_off = p->dev.win_off;
    a.n_tok = p->n_tok;
    a.nh = p->nh;
    a.C = C;
    a.nbins = p->nbins;
    for (int i = 0; i < 3; ++i) a.win[i] = p->d.window[i];
    a.tau = p->tau;
    const size_t dyn = 2 * (size_t)p->nbins * sizeof(float);
    for (const auto& r : p->bwd_ranges) {
      a.work = p->dev.bwd_work + r.begin;
      a.item_base = r.begin;
      kBwd[r.nqt](a, r.count, p->nh, dyn, s);
    }
    e = hipGetLastError();
    if (e == hipSuccess) e = trace_mark(s);
    if (e != hipSuccess) return e;
    const int per_item = p->nh * p->nbins;
    k_dbias_reduce<<<(unsigned)((per_item + 255) / 256), 256, 0, s>>>(dbias_part, (int)p->bwd_work.size(), per_item,
                                                                       dtable);
    e = hipGetLastError();
    if (e == hipSuccess) e = trace_mark(s);
  }
  if (e != hipSuccess) return e;
  // QKV backward: dx = scatter(dqkv W_qkv), dW_qkv = dqkv^T gather(x), db_qkv
  e = launch_dgrad_qkv_bf16(p, dqkv, wqkvT, dx, dx32, s);
  if (e == hipSuccess) e = trace_mark(s);
  if (e == hipSuccess)
    e = launch_wgrad_bf16(dqkv, 3 * C, (const bf16*)x, C, p->n_tok, 3 * C, C, p->wgrad_splits_qkv,
                          p->wgrad_chunk_qkv, part, dw_qkv, db_qkv, s);
  if (e == hipSuccess) e = trace_mark(s);
  return e;
}

}  // namespace swin
