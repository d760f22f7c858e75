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
// of the chunk. A window's Q, K and V (n x 32 bf16 each) are staged in LDS by direct
// global->LDS copies into one of two buffers, so the copies for window w+1 run while
// window w is computed (one barrier per window).
//
// The logits are computed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16), so a lane
// holds one query and 4 consecutive keys of every 16-key tile. The row max is an
// in-register reduction plus two cross-lane steps; the row sum comes from the matrix core
// (an all-ones operand against the same bf16 P as the PV product); and the probabilities
// of two adjacent key tiles are already the B operand of O^T = V^T P^T. The V^T operand is
// read from the row-major V tile with gfx950's transposing LDS read. A window has at most
// 256 tokens, so a query's whole key row lives in registers and the softmax is exact in a
// single pass (no online rescaling).
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
  static constexpr int ROWS = (NKT + 1) / 2 * 32;      // staged rows per tile (32-key chunks)
  static constexpr int FROWS = (ROWS + 63) / 64 * 64;  // word rows: whole 64-lane copies
  unsigned char q[ROWS * 64], k[ROWS * 64], v[ROWS * 64];
  int grow[FROWS];  // grid row of each token of the window
};

template <int NKT>
__global__ __launch_bounds__(64 * NKT, 1) void k_attn_fwd(AttnArgs a) {
  constexpr int NKC = (NKT + 1) / 2;   // 32-key chunks of the PV product
  constexpr int ROWS = FwdBuf<NKT>::ROWS;
  // Two buffers, filled by direct global->LDS copies: window w is computed from one while
  // window w+1 is copied into the other. They are separate objects (and the window loop is
  // unrolled by two) so the compiler can tell the copies never touch the buffer being read
  // and leaves them in flight until the end-of-window barrier.
  __shared__ __attribute__((aligned(1024))) FwdBuf<NKT> bufA;
  __shared__ __attribute__((aligned(1024))) FwdBuf<NKT> bufB;
  __shared__ int offs[kMaxChunk];
  __shared__ int codes[16 * NKT];     // per-token local-offset codes and wrap labels
  extern __shared__ float tab_lds[];  // [nbins]: the head's bias table times log2(e)

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
  for (int i = threadIdx.x; i < a.nbins; i += 64 * NKT) tab_lds[i] = tab[i] * kLog2e;
  if (threadIdx.x < wk.count) offs[threadIdx.x] = a.win_off[a.class_win[wk.first + threadIdx.x]];
  if (threadIdx.x < 16 * NKT) codes[threadIdx.x] = threadIdx.x < n ? token_code(threadIdx.x, ci.ext, ci.split, a.win) : 0;
  const int64_t off0 = a.win_off[a.class_win[wk.first]];

  const bf16* Qh = a.qkv + ((int64_t)(0 * a.nh + h) * a.n_tok) * 32;
  const bf16* Kh = a.qkv + ((int64_t)(1 * a.nh + h) * a.n_tok) * 32;
  const bf16* Vh = a.qkv + ((int64_t)(2 * a.nh + h) * a.n_tok) * 32;
  // rows past n arrive as zeros (buffer range = the window's n rows)
  auto stage = [&](int64_t off, FwdBuf<NKT>& b) {
    const uint32_t bytes = (uint32_t)n * 64;
    stage_rows(make_rsrc(Qh + off * 32, bytes), b.q, ROWS, qt, NKT, lane);
    stage_rows(make_rsrc(Kh + off * 32, bytes), b.k, ROWS, qt, NKT, lane);
    stage_rows(make_rsrc(Vh + off * 32, bytes), b.v, ROWS, qt, NKT, lane);
    stage_floats(make_rsrc(a.perm + off, (uint32_t)n * 4), (float*)b.grow, FwdBuf<NKT>::FROWS, qt, NKT, lane);
  };
  stage(off0, bufA);
  __syncthreads();  // table and offsets in LDS

  // bias + mask of this lane's query against every key; keys past n are masked, and
  // queries past n (whose outputs are dropped) get finite zeros
  const int code0 = code0_of(a.win);
  const int cq = codes[q];
  f32x4 bias[NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    const int4 ck = *(const int4*)(codes + 16 * kt + 4 * g);
    const int kk[4] = {ck.x, ck.y, ck.z, ck.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = 16 * kt + 4 * g + i;
      bias[kt][i] = !qv ? 0.f : (k >= n ? -INFINITY : pair_bias_codes(cq, kk[i], code0, tab_lds));
    }
  }
  __syncthreads();

  // a window's results are stored at the start of the next iteration, after the next
  // copies are issued, so the end-of-window barrier does not wait for them
  bf16x4 ov[2] = {};
  float lse_v = 0.f;
  int64_t prev_off = -1;
  int prev_row = 0;  // grid row of this lane's query in the previous window
  auto flush = [&]() {
    if (prev_off >= 0 && qv) {
      bf16* orow = a.o + (int64_t)prev_row * a.C + h * 32;
      *(bf16x4*)(orow + 4 * g) = ov[0];
      *(bf16x4*)(orow + 16 + 4 * g) = ov[1];
      if (g == 0) a.lse[(int64_t)h * a.n_tok + prev_off + q] = lse_v;
    }
  };
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = to_bf16(1.f);
  auto window = [&](int w, const FwdBuf<NKT>& cur, FwdBuf<NKT>& nxt) {
    const int64_t off = offs[w];
    if (w + 1 < wk.count) stage(offs[w + 1], nxt);  // overlaps with this window's compute
    flush();
    const bf16x8 bq = tile_frag(cur.q, q, g);
    f32x4 s[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) s[kt] = mfma16(tile_frag(cur.k, 16 * kt + li, g), bq, bias[kt]);
    float m = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, s[kt][i]);
    m = wave_max_xor16_32(m);
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[kt][i] = fast_exp2(s[kt][i] - m);

    // O^T = V^T P^T, and the row sums of the same bf16 P from an all-ones A operand: every row
    // of that product is the lane's query sum, so no cross-lane reduction is needed
    f32x4 oacc[2] = {f32x4{}, f32x4{}};
    f32x4 lacc = f32x4{};
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = to_bf16(s[2 * c][i]);
        pb[4 + i] = (2 * c + 1 < NKT) ? to_bf16(s[2 * c + 1][i]) : to_bf16(0.f);
      }
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) oacc[dt] = mfma16(tile_frag_tr(cur.v, 32 * c, 16 * dt, g, li), pb, oacc[dt]);
      lacc = mfma16(ones, pb, lacc);
    }
    const float l = lacc[0];
    const float inv = 1.f / l;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[dt][i] = to_bf16(oacc[dt][i] * inv);
    lse_v = m + fast_log2(l);
    prev_off = off;
    prev_row = cur.grow[q];
    __syncthreads();  // window w+1 staged; this buffer is free
  };
  for (int w = 0; w < wk.count; w += 2) {
    window(w, bufA, bufB);
    if (w + 1 < wk.count) window(w + 1, bufB, bufA);
  }
  flush();
}

template <int NKT>
static void launch_one(const AttnArgs& a, int n_items, int nh, hipStream_t s) {
  k_attn_fwd<NKT><<<dim3((unsigned)n_items, (unsigned)nh), 64 * NKT, (size_t)a.nbins * sizeof(float), s>>>(a);
}

typedef void (*fwd_launcher)(const AttnArgs&, int, int, hipStream_t);
static const fwd_launcher kFwd[17] = {nullptr,          launch_one<1>,  launch_one<2>,  launch_one<3>,
                                      launch_one<4>,    launch_one<5>,  launch_one<6>,  launch_one<7>,
                                      launch_one<8>,    launch_one<9>,  launch_one<10>, launch_one<11>,
                                      launch_one<12>,   launch_one<13>, launch_one<14>, launch_one<15>,
                                      launch_one<16>};

hipError_t launch_attn_fwd_bf16(const swin_attn_plan* p, const void* qkv, const float* table, void* o, float* lse,
                                hipStream_t s) {
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
