// Tiled window attention (bf16 MFMA, fp32 softmax) for windows of any size and head_dim
// 32, 64 or 128: the same module as attn_fwd.hip / attn_bwd.hip, for the windows that do not
// fit one tile (more than 256 tokens; TERRA section VII-A switches to FlashAttention from
// w >= 32, and BEAST's models use windows of thousands of tokens) and for wider heads
// (TERRA Table V: head_dim 128).
//
// Forward: one workgroup per (window, block of 64 queries, head), a wave per 16 queries. The
// window's keys and values stream through LDS in blocks of 64 rows, double-buffered by direct
// global->LDS copies, and the softmax is the online one: per block the running row max m,
// row sum l and output accumulator are rescaled by exp2(m_old - m_new). Logits are computed
// transposed (S^T = K Q^T, v_mfma_f32_16x16x32_bf16), so a lane holds one query and 4 keys of
// every 16-key tile, and its probabilities are directly the B operand of O^T = V^T P^T (the
// V^T operand comes from the transposing LDS read); the row sums come from the matrix core
// (an all-ones operand against the same bf16 P). Bias + mask come from the tokens' local
// offset codes and the head's relative-position table in global memory.
#include "device_common.h"
#include "swin_internal.h"

namespace swin {

constexpr int kTB = 64;  // tokens per query / key block

struct TiledArgs {
  const bf16* qkv;          // [3][nh][n_tok][hd], window-major rows
  const float* table;       // [nh][nbins]
  bf16* o;                  // [n_tok][C], grid order
  const int32_t* perm;      // window-major slot -> grid row
  float* lse;               // [nh][n_tok], log2 units
  const WorkItem* work;     // (class, window, block)
  const ClassInfo* classes;
  const int32_t* win_off;
  int64_t n_tok;
  int nh, C, nbins;
  int win[3];
  // backward
  const bf16* dO;           // [nh][n_tok][hd] window-major
  const float* dd;          // -D = -rowsum(dO o), [nh][n_tok]
  bf16* dqkv;               // [n_tok][3C], grid order
  unsigned long long* dbias_acc;  // [nh][nbins] fixed point (2^-32 units, two's complement)
  float tau;
};

// Token codes of keys past the window's end: a wrap label no real token has, so every pair
// with them is masked.
constexpr int kPadCode = 0x7f << 24;

template <int HD>
struct TiledBuf {
  unsigned char k[HD / 32][kTB * 64];  // 32-column sub-tiles of the block, swizzled 64-byte rows
  unsigned char v[HD / 32][kTB * 64];
  int codes[kTB];
};

template <int HD>
struct TiledFwdSmem {
  TiledBuf<HD> buf[2];
};

// Copies rows [kb*64, kb*64 + 64) of the planes a and b of one window (rows past n repeat row
// n-1) into the sub-tiles of buffer dst; wave wv issues HD/32 copies per plane. Threads < 64
// also write the keys' codes.
template <int HD>
__device__ __forceinline__ void tiled_stage(const bf16* a, const bf16* b, int64_t off, int n, int kb, int wv,
                                            int lane, const ClassInfo& ci, const int* win, unsigned char (*da)[kTB * 64],
                                            unsigned char (*db)[kTB * 64], int* codes) {
  constexpr int NSUB = HD / 32;
#pragma unroll
  for (int t = 0; t < NSUB; ++t) {
    const int i = wv + 4 * t;
    const int c = i >> 2, j = i & 3;
    const int row = 16 * j + (lane >> 2);
    const int key = kb * kTB + row;
    const int src_row = key < n ? key : n - 1;
    const int lc = (lane & 3) ^ swz(row);
    const int64_t src = (off + src_row) * HD + 32 * c + 8 * lc;
    lds_copy16(a + src, da[c] + 1024 * j);
    if (db) lds_copy16(b + src, db[c] + 1024 * j);
  }
  if (codes && wv == 0) {
    const int key = kb * kTB + lane;
    codes[lane] = key < n ? token_code(key, ci.ext, ci.split, win) : kPadCode;
  }
}

// Bias + mask of a pair in log2 units, without branches: the table index is in range for
// every pair of real tokens and for a real query against a padding key (code 0 in the low
// bits; local codes never exceed code0), so the read is issued for all lanes and the label
// test selects -inf afterwards.
__device__ __forceinline__ float tiled_bias(int cq, int ck, int code0, const float* tab) {
  const float t = tab[(cq & 0xffffff) - (ck & 0xffffff) + code0];
  return (cq >> 24) != (ck >> 24) ? -INFINITY : t * kLog2e;
}

template <int HD>
__global__ __launch_bounds__(256, 2) void k_tiled_fwd(TiledArgs a) {
  constexpr int NSUB = HD / 32;
  __shared__ __attribute__((aligned(1024))) TiledFwdSmem<HD> sm;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, li = lane & 15;
  const WorkItem wk = a.work[blockIdx.x];
  const int h = blockIdx.y;
  const ClassInfo ci = a.classes[wk.cls];
  const int n = ci.n;
  const int64_t off = a.win_off[wk.first];
  const int q = wk.count * kTB + 16 * wv + li;  // window-local query of this lane
  const bool qv = q < n;
  const int qc = qv ? q : n - 1;
  const size_t plane = (size_t)a.nh * a.n_tok * HD;
  const bf16* Qh = a.qkv + (size_t)h * a.n_tok * HD;
  const bf16* Kh = Qh + plane;
  const bf16* Vh = Kh + plane;
  const float* tab = a.table + (int64_t)h * a.nbins;
  const int code0 = code0_of(a.win);
  const int cq = token_code(qc, ci.ext, ci.split, a.win);
  const int nkb = (n + kTB - 1) / kTB;

  tiled_stage<HD>(Kh, Vh, off, n, 0, wv, lane, ci, a.win, sm.buf[0].k, sm.buf[0].v, sm.buf[0].codes);
  // the lane's query: B operand of S^T = K Q^T, hd values 32 c + 8 g .. + 7
  bf16x8 bq[NSUB];
#pragma unroll
  for (int c = 0; c < NSUB; ++c) bq[c] = *(const bf16x8*)(Qh + (off + qc) * HD + 32 * c + 8 * g);
  // The fragments are laundered through empty asm after an explicit wait, here and for the
  // bias values below, so the compiler sees no load result in flight across the copies of the
  // next block (it would otherwise wait for those copies too before the first use).
  vm_wait(0);
#pragma unroll
  for (int c = 0; c < NSUB; ++c) asm volatile("" : "+v"(bq[c]));

  const int kq_off = li * 64 + 16 * (g ^ swz(li));
  const int vr = 4 * g + (li >> 2);
  const int vt_off0 = swz_off(vr, 4 * (li & 3)), vt_off1 = swz_off(vr, 16 + 4 * (li & 3));
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = to_bf16(1.f);
  float m = -INFINITY, l = 0.f;
  f32x4 oacc[HD / 16];
#pragma unroll
  for (int d = 0; d < HD / 16; ++d) oacc[d] = f32x4{};

  for (int kb = 0; kb < nkb; ++kb) {
    // this wave's copies of block kb have landed (no other vector-memory operation is in
    // flight here); the barrier then covers every wave's copies and codes, and every wave is
    // done with the buffer the next block goes to
    vm_wait(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const TiledBuf<HD>& cur = sm.buf[kb & 1];
    // bias + mask first: its table reads finish before the next block's copies are issued,
    // so waiting for them never waits for those copies
    f32x4 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int4 ck = *(const int4*)(cur.codes + 16 * kt + 4 * g);
      const int kk[4] = {ck.x, ck.y, ck.z, ck.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float b = tiled_bias(cq, kk[i], code0, tab);
        s[kt][i] = qv ? b : 0.f;
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) asm volatile("" : "+v"(s[kt]));
    if (kb + 1 < nkb) {
      TiledBuf<HD>& nx = sm.buf[(kb + 1) & 1];
      tiled_stage<HD>(Kh, Vh, off, n, kb + 1, wv, lane, ci, a.win, nx.k, nx.v, nx.codes);
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int c = 0; c < NSUB; ++c) s[kt] = mfma16(*(const bf16x8*)(cur.k[c] + kq_off + 1024 * kt), bq[c], s[kt]);
    float mb = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mb = fmaxf(mb, s[kt][i]);
    mb = wave_max_xor16_32(mb);
    const float mn = fmaxf(m, mb);
    const float ms = mn == -INFINITY ? 0.f : mn;  // nothing allowed yet: keep every term at 0
    const float corr = fast_exp2(m - ms);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[kt][i] = fast_exp2(s[kt][i] - ms);
#pragma unroll
    for (int d = 0; d < HD / 16; ++d) oacc[d] *= corr;
    f32x4 lacc = f32x4{};
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = to_bf16(s[2 * cc][i]);
        pb[4 + i] = to_bf16(s[2 * cc + 1][i]);
      }
#pragma unroll
      for (int sc = 0; sc < NSUB; ++sc) {
        bf16x8 v0, v1;
        tile_frag_tr2_at(cur.v[sc] + 2048 * cc, vt_off0, vt_off1, v0, v1);
        oacc[2 * sc] = mfma16(v0, pb, oacc[2 * sc]);
        oacc[2 * sc + 1] = mfma16(v1, pb, oacc[2 * sc + 1]);
      }
      lacc = mfma16(ones, pb, lacc);
    }
    l = l * corr + lacc[0];
    m = mn;
  }
  if (qv) {
    const float inv = __builtin_amdgcn_rcpf(l);
    const int64_t grow = a.perm[off + q];
    bf16* orow = a.o + grow * a.C + (int64_t)h * HD;
#pragma unroll
    for (int sc = 0; sc < NSUB; ++sc) {
      bf16x4 o0, o1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o0[i] = to_bf16(oacc[2 * sc][i] * inv);
        o1[i] = to_bf16(oacc[2 * sc + 1][i] * inv);
      }
      *(bf16x4*)(orow + 32 * sc + 4 * g) = o0;
      *(bf16x4*)(orow + 32 * sc + 16 + 4 * g) = o1;
    }
    if (g == 0) a.lse[(int64_t)h * a.n_tok + off + q] = m + fast_log2(l);
  }
}

static TiledArgs tiled_args(const swin_attn_plan* p) {
  TiledArgs a{};
  a.perm = p->dev.perm;
  a.work = p->dev.tiled_work;
  a.classes = p->dev.classes;
  a.win_off = p->dev.win_off;
  a.n_tok = p->n_tok;
  a.nh = p->nh;
  a.C = p->C;
  a.nbins = p->nbins;
  for (int i = 0; i < 3; ++i) a.win[i] = p->d.window[i];
  a.tau = p->tau;
  return a;
}

hipError_t launch_tiled_fwd_bf16(const swin_attn_plan* p, const void* qkv, const float* table, void* o, float* lse,
                                 hipStream_t s) {
  TiledArgs a = tiled_args(p);
  a.qkv = (const bf16*)qkv;
  a.table = table;
  a.o = (bf16*)o;
  a.lse = lse;
  const dim3 grid((unsigned)p->tiled_work.size(), (unsigned)p->nh);
  if (p->hd == 32)
    k_tiled_fwd<32><<<grid, 256, 0, s>>>(a);
  else if (p->hd == 64)
    k_tiled_fwd<64><<<grid, 256, 0, s>>>(a);
  else
    k_tiled_fwd<128><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace swin
