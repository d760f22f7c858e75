// Tiled window attention (bf16 MFMA, fp32 softmax) for windows of any size and head_dim
// 32, 64 or 128: the same module as attn_fwd.hip / attn_bwd.hip, for the windows that do not
// fit one tile (more than 256 tokens; TERRA section VII-A switches to FlashAttention from
// w >= 32, and BEAST's models use windows of thousands of tokens) and for wider heads
// (TERRA Table V: head_dim 128).
//
// Forward (k_tiled_fwd_pipe): one workgroup per (window, block of 128 queries, head), a wave
// per 32 queries. The window's keys and values stream through LDS in blocks of 64 rows
// (buffer loads straight to LDS), and the softmax is the online one with a lazily moved
// exponent offset. Logits are computed transposed (S^T = K Q^T, v_mfma_f32_32x32x16_bf16), so
// a lane holds one query and 32 keys of each block, and its probabilities are directly the B
// operand of O^T = V^T P^T (the V^T operand comes from the transposing LDS read). Bias + mask
// come from per-class token-code tables and the head's relative-position table (fp16 in LDS
// when it has at most kTabLds bins, else fp32 in global memory).
//
// Backward (recomputing P from q, k and the saved LSE; dS = P (dP - D), D = rowsum(dO o)):
//   k_tiled_bwd_dkv: one workgroup per (window, block of 128 keys, head), a wave per 16 keys;
//     query blocks (q, dO, LSE, -D, codes) stream through LDS; dV^T += dO^T P and
//     dK^T += q^T dS accumulate in registers; dT is binned per workgroup in LDS as 64-bit
//     fixed point (units of 2^-20), then added to a global fixed-point accumulator. Integer
//     sums do not depend on the order of the additions, so dT is bitwise reproducible.
//   k_tiled_bwd_dq: one workgroup per (window, block of 64 queries, head), a wave per 16
//     queries on v_mfma_f32_16x16x32_bf16: key blocks stream through LDS and dQ^T += K^T dS^T.
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
  const WorkItem* work;     // (class, window, 64-token block)
  const WorkItem* kv_work;  // (class, window, 128-token block): the dK/dV kernel's items
  const ClassInfo* classes;
  const int32_t* win_off;
  int64_t n_tok;
  int nh, C, nbins;
  int win[3];
  const int32_t* codes;     // per class: key codes, then query codes (see kCodeRound)
  // backward
  const bf16* dO;           // [nh][n_tok][hd] window-major
  const float* dd;          // -D = -rowsum(dO o), [nh][n_tok]
  bf16* dqkv;               // [n_tok][3C], grid order
  unsigned long long* dbias_acc;  // [nh][nbins] fixed point (units of 1/kFix, two's complement)
  float tau;
};

template <int HD>
struct TiledBuf {
  unsigned char k[HD / 32][kTB * 64];  // 32-column sub-tiles of the block, swizzled 64-byte rows
  unsigned char v[HD / 32][kTB * 64];
  int codes[kTB];
};

// Fills the LDS table (bins, then -inf) when it fits; made visible by the first barrier.
__device__ __forceinline__ void tiled_tab_fill(_Float16* dst, const float* tab, int nbins, int nthreads) {
  if (nbins > kTabLds) return;
  for (int i = threadIdx.x; i <= nbins; i += nthreads)
    dst[i] = i < nbins ? (_Float16)(tab[i] * kLog2e) : (_Float16)(-INFINITY);
}

// LDS of the dQ kernel. The table comes first so that its reads take their base from the
// instruction's offset field.
template <int HD>
struct TiledFwdSmem {
  _Float16 tab[kTabLds + 8];
  alignas(1024) TiledBuf<HD> buf[2];
};

// Copy of rows [kb*64, kb*64 + 64) of one window's plane into the swizzled 32-column sub-tiles
// dst[c] through buffer loads straight to LDS. The resource spans the window's n rows, so rows
// past n arrive as zeros. The 4 HD/32 one-kilobyte copies are spread over the NW waves (NW a
// multiple of 4): wave w copies the 16-row slab w % 4 of sub-tiles w/4 + NW/4 t. voff is the
// lane's byte offset inside a block (stage_voff).
template <int HD, int NW>
__device__ __forceinline__ void stage_plane(__amdgpu_buffer_rsrc_t src, int kb, int wv, uint32_t voff,
                                            unsigned char (*dst)[kTB * 64]) {
  constexpr int NSUB = HD / 32;
  constexpr int PER = (4 * NSUB + NW - 1) / NW;
  static_assert(NW % 4 == 0, "whole slabs per wave");
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const int c = (wv >> 2) + (NW / 4) * t;
    if ((4 * NSUB) % NW != 0 && c >= NSUB) break;  // wave-uniform
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)(dst[c] + 1024 * (wv & 3)),
                                             16, voff + (uint32_t)(kb * kTB * HD * 2 + 64 * c), 0, 0, 0);
  }
}
// Lane offset of stage_plane: row 16 (w % 4) + lane/4 of the block, logical 16-byte chunk
// (lane % 4) ^ swz(row) of each 32-column sub-tile (the chunk lands in slot lane % 4).
template <int HD>
__device__ __forceinline__ uint32_t stage_voff(int wv, int lane) {
  const int row = 16 * (wv & 3) + (lane >> 2);
  return (uint32_t)(row * HD * 2 + 16 * ((lane & 3) ^ swz(row)));
}
// Dwords [kb*64, kb*64 + 64) of a per-token table (codes, LSE, -D; resource over the window's
// or class's entries, zeros past them) into 64 consecutive LDS dwords.
__device__ __forceinline__ void stage_dwords(__amdgpu_buffer_rsrc_t src, int kb, int lane, void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)dst, 4,
                                           (uint32_t)(4 * (kb * kTB + lane)), 0, 0, 0);
}

// Bias + mask of a pair in log2 units, without branches: the table index is in range for
// every pair of real tokens and for a real query against a padding key (code 0 in the low
// bits; local codes never exceed code0), so the read is issued for all lanes and the label
// test selects -inf afterwards.
__device__ __forceinline__ float tiled_bias(int cq, int ck, int code0, const float* tab) {
  const float t = tab[(cq & 0xffffff) - (ck & 0xffffff) + code0];
  return (cq >> 24) != (ck >> 24) ? -INFINITY : t * kLog2e;
}

// Four transposing reads for 32x32x16 V^T operands: f0 = the rows at offa and offb (keys
// 4 hh + i/4 and 8 + 4 hh + i/4 of a 16-key step), f1 = the rows 16 further (the next step);
// ended by their own LDS wait (see tile_frag_tr2_at).
__device__ __forceinline__ void tile_frag_tr32(const unsigned char* tile, int offa, int offb, bf16x8& f0,
                                               bf16x8& f1) {
  const uint32_t base = lds_addr(tile);
  u32x2 v0, v1, v2, v3;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %4 offset:1024\n\t"
      "ds_read_b64_tr_b16 %3, %5 offset:1024\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
      : "v"(base + offa), "v"(base + offb)
      : "memory");
  f0 = __builtin_bit_cast(bf16x8, u32x4{v0[0], v0[1], v1[0], v1[1]});
  f1 = __builtin_bit_cast(bf16x8, u32x4{v2[0], v2[1], v3[0], v3[1]});
}

// Forward with 32 queries per wave: 4 waves, 128-query blocks, S^T = K Q^T and O^T = V^T P^T
// on v_mfma_f32_32x32x16_bf16. A lane holds one query (lane % 32) and 32 keys of each 64-key
// block (rows 32 t + 8 j + 4 hh + i, hh = lane / 32), so every K and V fragment read from LDS
// serves 32 queries. The exponent offset m moves only when a block's maximum exceeds it by
// more than kRescale (log2 units), so most blocks skip the rescaling of O; the probabilities
// then lie in [0, 2^kRescale] and the final normalisation is unchanged. The bias enters the S
// accumulator already shifted by -m (one mixed-precision FMA per pair), and the row sums are
// taken from the same bf16 probabilities as the PV product (bf16 dot products).
constexpr float kRescale = 8.f;

// LDS of the pipelined forward: K runs one block ahead of V, codes two (ring of four).
template <int HD>
struct FwdPipeSmem {
  _Float16 tab[kTabLds + 8];
  alignas(1024) unsigned char k[2][HD / 32][kTB * 64];
  unsigned char v[2][HD / 32][kTB * 64];
  int codes[4][kTB];
};

// The forward, software-pipelined so that each wave's matrix and vector work
// overlap: in step kb the S MFMAs of block kb+1 run beside the exponentials of block kb, and the
// PV MFMAs of block kb beside the bias reads of block kb+2. Buffers: K(kb+1) and V(kb) are read
// in step kb while K(kb+2), V(kb+1) and the codes of block kb+3 are copied in.
// FAST: the bias table is in LDS (nbins <= kTabLds; the code tables are then encoded). The
// global-table variant needs more registers than two workgroups per CU leave at head_dim 128.
template <int HD, bool FAST>
__global__ __launch_bounds__(256, (FAST || HD < 128) ? 2 : 1) void k_tiled_fwd_pipe(TiledArgs a) {
  constexpr int NSUB = HD / 32;
  constexpr int KS = HD / 16;
  __shared__ __attribute__((aligned(1024))) FwdPipeSmem<HD> sm;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lq = lane & 31, hh = lane >> 5;
  const WorkItem wk = a.work[blockIdx.x];
  const int h = blockIdx.y;
  const ClassInfo ci = a.classes[wk.cls];
  const int n = ci.n;
  const int64_t off = a.win_off[wk.first];
  const int q = wk.count * 128 + 32 * wv + lq;
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
  const int qenc = qv ? enc_query(cq, code0) : kPadQ;
  const uint32_t lim = 2u * (uint32_t)a.nbins;
  const int nr = (n + kCodeRound - 1) / kCodeRound * kCodeRound;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + off * HD, (uint32_t)n * HD * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + off * HD, (uint32_t)n * HD * 2);
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.codes + wk.codes, (uint32_t)nr * 4);  // the class's key codes
  const uint32_t voff = stage_voff<HD>(wv, lane);
  const __amdgpu_buffer_rsrc_t rtab = make_rsrc(tab, (uint32_t)a.nbins * 4);  // global-table variant
  auto stage_k = [&](int j) { stage_plane<HD, 4>(rk, j, wv, voff, sm.k[j & 1]); };
  auto stage_v = [&](int j) { stage_plane<HD, 4>(rv, j, wv, voff, sm.v[j & 1]); };
  auto stage_c = [&](int j) {
    if (wv == 0) stage_dwords(rc, j, lane, sm.codes[j & 3]);
  };
  // bias - m of the lane's 32 keys of block j
  auto bias_init = [&](int j, float m_eff, f32x16 (&S)[2]) {
    if constexpr (FAST) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int4 ck = *(const int4*)(sm.codes[j & 3] + 32 * t + 8 * jj + 4 * hh);
          const int kk[4] = {ck.x, ck.y, ck.z, ck.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t ib = min((uint32_t)(qenc - kk[i]), lim);
            const uint32_t raw = *(const unsigned short*)((const char*)sm.tab + ib);
            S[t][4 * jj + i] = half_lo_minus(raw, m_eff);
          }
        }
    } else {
      // the head's table through a buffer resource (32-bit offsets), four pairs at a time
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int4 ck = *(const int4*)(sm.codes[j & 3] + 32 * t + 8 * jj + 4 * hh);
          const int kk[4] = {ck.x, ck.y, ck.z, ck.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t idx = (uint32_t)((cq & 0xffffff) - (kk[i] & 0xffffff) + code0);
            const float tv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rtab, 4 * idx, 0, 0));
            const float b = (cq >> 24) != (kk[i] >> 24) ? -INFINITY : tv * kLog2e;
            S[t][4 * jj + i] = (qv ? b : 0.f) - m_eff;
          }
        }
    }
  };

  tiled_tab_fill(sm.tab, tab, a.nbins, 256);
  stage_k(0);
  stage_c(0);
  if (nkb > 1) stage_c(1);
  bf16x8 bq[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) bq[s] = *(const bf16x8*)(Qh + (off + qc) * HD + 16 * s + 8 * hh);
  vm_wait(0);
#pragma unroll
  for (int s = 0; s < KS; ++s) asm volatile("" : "+v"(bq[s]));
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  const int k_off0 = lq * 64 + 16 * (hh ^ swz(lq)), k_off1 = lq * 64 + 16 * ((2 + hh) ^ swz(lq));
  const int i16 = lane & 15;
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);
  const int v_offa = swz_off(4 * hh + (i16 >> 2), vcol), v_offb = swz_off(8 + 4 * hh + (i16 >> 2), vcol);
  bf16x2 ones2;
  ones2[0] = to_bf16(1.f);
  ones2[1] = to_bf16(1.f);
  float m_run = -INFINITY, l = 0.f;
  f32x16 oacc[NSUB];
#pragma unroll
  for (int d = 0; d < NSUB; ++d) oacc[d] = f32x16{};

  auto s_mfma = [&](int j, f32x16 (&S)[2]) {
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        S[t] = mfma32(*(const bf16x8*)(sm.k[j & 1][s >> 1] + 2048 * t + ((s & 1) ? k_off1 : k_off0)), bq[s], S[t]);
  };

  // prologue: S(0) complete, bias of block 1 in Sb; K(1), V(0) and the codes of block 2 in flight
  f32x16 Sa[2], Sb[2];
  bias_init(0, 0.f, Sa);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (nkb > 1) stage_k(1);
  stage_v(0);
  if (nkb > 2) stage_c(2);
  s_mfma(0, Sa);
  if (nkb > 1) bias_init(1, 0.f, Sb);

  // one step: Sc = S(kb) (complete), Sn = bias(kb+1) - m; ends with Sc = bias(kb+2) - m and
  // Sn = S(kb+1) complete
  auto step = [&](int kb, f32x16 (&Sc)[2], f32x16 (&Sn)[2]) {
    vm_wait(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (kb + 2 < nkb) stage_k(kb + 2);
    if (kb + 1 < nkb) stage_v(kb + 1);
    if (kb + 3 < nkb) stage_c(kb + 3);
    const float m_old = m_run == -INFINITY ? 0.f : m_run;
    float mb = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mb = fmaxf(mb, Sc[t][r]);
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const bool need = mb > kRescale || (m_run == -INFINITY && mb != -INFINITY);
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float d = need ? mb : 0.f;
      const float corr = fast_exp2(-d);
#pragma unroll
      for (int dd = 0; dd < NSUB; ++dd) oacc[dd] *= corr;
      l *= corr;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          Sc[t][r] -= d;
          Sn[t][r] -= d;
        }
      m_run = need ? m_old + d : m_run;
    }
    // S(kb+1) on the matrix cores beside P(kb) on the vector ALUs. Past the last block both run
    // on stale buffers (in-bounds LDS reads, results unused), so no branch splits the step.
    s_mfma(kb + 1, Sn);
    bf16x8 pb[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[t][u][i] = to_bf16(fast_exp2(Sc[t][8 * u + i]));
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          l = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[t][u][2 * e], pb[t][u][2 * e + 1]}, ones2, l, false);
    // PV(kb) beside the bias of block kb+2
    const float m_eff = m_run == -INFINITY ? 0.f : m_run;
    // stale codes only address the LDS table (clamped); the global table needs the guard
    if (FAST || kb + 2 < nkb) bias_init(kb + 2, m_eff, Sc);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int sc = 0; sc < NSUB; ++sc) {
        bf16x8 f0, f1;
        tile_frag_tr32(sm.v[kb & 1][sc] + 2048 * t, v_offa, v_offb, f0, f1);
        oacc[sc] = mfma32(f0, pb[t][0], oacc[sc]);
        oacc[sc] = mfma32(f1, pb[t][1], oacc[sc]);
      }
  };
  for (int kb = 0; kb < nkb; kb += 2) {
    step(kb, Sa, Sb);
    if (kb + 1 < nkb) step(kb + 1, Sb, Sa);
  }
  l += __shfl_xor(l, 32);
  {
    // lanes l and l ^ 32 (same query) hold columns 8 j + 4 hh .. + 3 of every 32-column block;
    // they swap halves so that each writes two 16-byte pieces: columns 8 hh + 16 p .. + 7
    // (every lane takes part)
    const float inv = __builtin_amdgcn_rcpf(l);
    const int64_t grow = qv ? a.perm[off + q] : 0;
    bf16* orow = a.o + grow * a.C + (int64_t)h * HD + 8 * hh;
#pragma unroll
    for (int sc = 0; sc < NSUB; ++sc) {
      bf16x4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[j][i] = to_bf16(oacc[sc][4 * j + i] * inv);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const u32x2 send = __builtin_bit_cast(u32x2, hh ? v[2 * p] : v[2 * p + 1]);
        u32x2 recv;
        recv[0] = (uint32_t)__shfl_xor((int)send[0], 32);
        recv[1] = (uint32_t)__shfl_xor((int)send[1], 32);
        const bf16x4 r = __builtin_bit_cast(bf16x4, recv);
        const bf16x4 lo = hh ? r : v[2 * p], hi = hh ? v[2 * p + 1] : r;
        const bf16x8 o8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if (qv) *(bf16x8*)(orow + 32 * sc + 16 * p) = o8;
      }
    }
    if (qv && hh == 0) a.lse[(int64_t)h * a.n_tok + off + q] = m_run + fast_log2(l);
  }
}

// ---------------------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------------------
// dT is summed in fixed point: every dS term is rounded to a 32-bit integer in units of 2^-20
// and added into 64-bit integer bins, so the sums are exact and do not depend on the order of
// the additions. A term of magnitude 2^11 or more (or not a number) does not fit: it is clamped
// to +-kFixLim before the conversion, and the call's saturation word (the u64 after the
// accumulator) is set; the conversion to fp32 then writes NaN over the whole table and raises
// SWIN_FLAG_DT_SATURATED in the plan's sticky flags.
constexpr float kFix = 1048576.f;         // 2^20
constexpr float kFixLim = 2147483520.f;   // the largest float below 2^31

template <int HD>
struct TiledQBuf {
  unsigned char q[HD / 32][kTB * 64];
  unsigned char d[HD / 32][kTB * 64];  // dO
  float lse[kTB];
  float nd[kTB];                       // -D
  int codes[kTB];
};

// All of the dK/dV kernel's LDS is one static object: with one object the compiler leaves the
// ordering of the direct-to-LDS copies against LDS reads to the explicit waits.
template <int HD>
struct DkvSmem {
  _Float16 tab[kTabLds + 8];  // first: its reads and the bin additions keep small offsets
  unsigned long long bins[kTiledMaxBwdBins + 8];  // entry nbins: the masked pairs' (zero) terms
  alignas(1024) TiledQBuf<HD> buf[2];
};

// dQ: the forward's structure with lse fixed; dP^T = V dO^T starts from -D.
template <int HD, bool FAST>
__global__ __launch_bounds__(256, 2) void k_tiled_bwd_dq(TiledArgs a) {
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
  const int q = wk.count * kTB + 16 * wv + li;
  const bool qv = q < n;
  const int qc = qv ? q : n - 1;
  const size_t plane = (size_t)a.nh * a.n_tok * HD;
  const bf16* Qh = a.qkv + (size_t)h * a.n_tok * HD;
  const bf16* Kh = Qh + plane;
  const bf16* Vh = Kh + plane;
  const bf16* dOh = a.dO + (size_t)h * a.n_tok * HD;
  const float* tab = a.table + (int64_t)h * a.nbins;
  const int code0 = code0_of(a.win);
  const int cq = token_code(qc, ci.ext, ci.split, a.win);
  const int nkb = (n + kTB - 1) / kTB;
  const int qenc = qv ? enc_query(cq, code0) : kPadQ;
  const uint32_t lim = 2u * (uint32_t)a.nbins;

  tiled_tab_fill(sm.tab, tab, a.nbins, 256);
  const int nr = (n + kCodeRound - 1) / kCodeRound * kCodeRound;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + off * HD, (uint32_t)n * HD * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + off * HD, (uint32_t)n * HD * 2);
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.codes + wk.codes, (uint32_t)nr * 4);  // the class's key codes
  const uint32_t voff = stage_voff<HD>(wv, lane);
  auto stage = [&](int j, TiledBuf<HD>& b) {
    stage_plane<HD, 4>(rk, j, wv, voff, b.k);
    stage_plane<HD, 4>(rv, j, wv, voff, b.v);
    if (wv == 0) stage_dwords(rc, j, lane, b.codes);
  };
  stage(0, sm.buf[0]);
  bf16x8 bq[NSUB], bd[NSUB];
#pragma unroll
  for (int c = 0; c < NSUB; ++c) {
    bq[c] = *(const bf16x8*)(Qh + (off + qc) * HD + 32 * c + 8 * g);
    bd[c] = *(const bf16x8*)(dOh + (off + qc) * HD + 32 * c + 8 * g);
  }
  float lse_q = a.lse[(int64_t)h * a.n_tok + off + qc];
  float nd_q = a.dd[(int64_t)h * a.n_tok + off + qc];
  vm_wait(0);
#pragma unroll
  for (int c = 0; c < NSUB; ++c) asm volatile("" : "+v"(bq[c]), "+v"(bd[c]));
  asm volatile("" : "+v"(lse_q), "+v"(nd_q));

  const int kq_off = li * 64 + 16 * (g ^ swz(li));
  const int vr = 4 * g + (li >> 2);
  const int kt_off0 = swz_off(vr, 4 * (li & 3)), kt_off1 = swz_off(vr, 16 + 4 * (li & 3));
  f32x4 dqacc[HD / 16];
#pragma unroll
  for (int d = 0; d < HD / 16; ++d) dqacc[d] = f32x4{};

  for (int kb = 0; kb < nkb; ++kb) {
    vm_wait(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const TiledBuf<HD>& cur = sm.buf[kb & 1];
    f32x4 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int4 ck = *(const int4*)(cur.codes + 16 * kt + 4 * g);
      const int kk[4] = {ck.x, ck.y, ck.z, ck.w};
      if constexpr (FAST) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // bias - lse; queries past n: -inf
          const uint32_t ib = min((uint32_t)(qenc - kk[i]), lim);
          s[kt][i] = half_lo_minus(*(const unsigned short*)((const char*)sm.tab + ib), lse_q);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float b = tiled_bias(cq, kk[i], code0, tab);
          s[kt][i] = qv ? b - lse_q : -INFINITY;  // queries past n: P = 0, nothing flows back
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) asm volatile("" : "+v"(s[kt]) : : "memory");
    if (kb + 1 < nkb) {
      TiledBuf<HD>& nx = sm.buf[(kb + 1) & 1];
      stage(kb + 1, nx);
    }
    f32x4 ds[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int c = 0; c < NSUB; ++c) s[kt] = mfma16(*(const bf16x8*)(cur.k[c] + kq_off + 1024 * kt), bq[c], s[kt]);
      f32x4 dp = {nd_q, nd_q, nd_q, nd_q};
#pragma unroll
      for (int c = 0; c < NSUB; ++c) dp = mfma16(*(const bf16x8*)(cur.v[c] + kq_off + 1024 * kt), bd[c], dp);
#pragma unroll
      for (int i = 0; i < 4; ++i) ds[kt][i] = fast_exp2(s[kt][i]) * dp[i];
    }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      bf16x8 db;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        db[i] = to_bf16(ds[2 * cc][i]);
        db[4 + i] = to_bf16(ds[2 * cc + 1][i]);
      }
#pragma unroll
      for (int sc = 0; sc < NSUB; ++sc) {
        bf16x8 k0, k1;
        tile_frag_tr2_at(cur.k[sc] + 2048 * cc, kt_off0, kt_off1, k0, k1);
        dqacc[2 * sc] = mfma16(k0, db, dqacc[2 * sc]);
        dqacc[2 * sc + 1] = mfma16(k1, db, dqacc[2 * sc + 1]);
      }
    }
  }
  {
    // 16-byte pieces: lanes 16 apart (same query) swap halves (every lane takes part)
    const int64_t grow = qv ? a.perm[off + q] : 0;
    bf16* row = a.dqkv + grow * 3 * a.C + (int64_t)h * HD + pair_col(g);
#pragma unroll
    for (int sc = 0; sc < NSUB; ++sc) {
      bf16x4 o0, o1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o0[i] = to_bf16(dqacc[2 * sc][i] * a.tau);
        o1[i] = to_bf16(dqacc[2 * sc + 1][i] * a.tau);
      }
      const bf16x8 o8 = pair_cols(o0, o1, g);
      if (qv) *(bf16x8*)(row + 32 * sc) = o8;
    }
  }
}

// 64-bit integer add to LDS, as inline assembly: the compiler treats its own LDS atomics as
// possibly aliasing direct-to-LDS copies in flight and would wait for those copies first.
// The bins are touched only by these additions, by the zeroing before the first barrier and
// by the read-out after an explicit LDS wait and a barrier.
__device__ __forceinline__ void lds_add_u64(unsigned long long* p, uint64_t v) {
  asm volatile("ds_add_u64 %0, %1" : : "v"(lds_addr(p)), "v"(v));
}
__device__ __forceinline__ void lds_add_u64_at(uint32_t addr, uint64_t v) {
  asm volatile("ds_add_u64 %0, %1" : : "v"(addr), "v"(v));
}

constexpr int kKvWaves = 8;  // dK/dV: 8 waves of 16 keys, so two waves share each SIMD

// FAST: the bias table is in LDS (nbins <= kTabLds; the code tables are then encoded).
template <int HD, bool FAST>
__global__ __launch_bounds__(64 * kKvWaves, 1) void k_tiled_bwd_dkv(TiledArgs a) {
  constexpr int NW = kKvWaves;
  constexpr int NSUB = HD / 32;
  __shared__ __attribute__((aligned(1024))) DkvSmem<HD> sm;
  TiledQBuf<HD>* buf = sm.buf;
  unsigned long long* bins = sm.bins;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, li = lane & 15;
  const WorkItem wk = a.kv_work[blockIdx.x];
  const int h = blockIdx.y;
  const ClassInfo ci = a.classes[wk.cls];
  const int n = ci.n;
  const int64_t off = a.win_off[wk.first];
  const int k = wk.count * 16 * NW + 16 * wv + li;  // window-local key of this lane
  const bool kv = k < n;
  const int kc = kv ? k : n - 1;
  const size_t plane = (size_t)a.nh * a.n_tok * HD;
  const bf16* Qh = a.qkv + (size_t)h * a.n_tok * HD;
  const bf16* Kh = Qh + plane;
  const bf16* Vh = Kh + plane;
  const bf16* dOh = a.dO + (size_t)h * a.n_tok * HD;
  const float* tab = a.table + (int64_t)h * a.nbins;
  const int code0 = code0_of(a.win);
  // keys past n take the padding code: every pair masked, nothing accumulated
  const int ck = kv ? token_code(k, ci.ext, ci.split, a.win) : kPadCode;
  const int nqb = (n + kTB - 1) / kTB;
  const int kenc = kv ? enc_key(ck) : kPadK;
  const uint32_t lim = 2u * (uint32_t)a.nbins;

  // tables over kTiledMaxBwdBins bins (global-table variant only): every allowed pair's term goes
  // straight to the global accumulator (64-bit integer atomics: exact, order-free) and the LDS bins
  // stay unused
  const bool global_bins = !FAST && a.nbins > kTiledMaxBwdBins;
  unsigned long long* acc = a.dbias_acc + (int64_t)h * a.nbins;
  if (!global_bins)
    for (int i = threadIdx.x; i <= a.nbins; i += 64 * NW) bins[i] = 0ull;
  const uint32_t bins_base = lds_addr(bins);
  tiled_tab_fill(sm.tab, tab, a.nbins, 64 * NW);
  // query block j of q and dO (zeros past n) with its codes (the class's query codes follow its
  // key codes), LSE and -D
  const int nr = (n + kCodeRound - 1) / kCodeRound * kCodeRound;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qh + off * HD, (uint32_t)n * HD * 2);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(dOh + off * HD, (uint32_t)n * HD * 2);
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.codes + wk.codes + nr, (uint32_t)nr * 4);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.lse + (int64_t)h * a.n_tok + off, (uint32_t)n * 4);
  const __amdgpu_buffer_rsrc_t rn = make_rsrc(a.dd + (int64_t)h * a.n_tok + off, (uint32_t)n * 4);
  const uint32_t voff = stage_voff<HD>(wv, lane);
  auto stage_q = [&](int j, TiledQBuf<HD>& b) {
    stage_plane<HD, NW>(rq, j, wv, voff, b.q);
    stage_plane<HD, NW>(rd, j, wv, voff, b.d);
    if (wv == 0) stage_dwords(rc, j, lane, b.codes);
    if (wv == 1) {
      stage_dwords(rl, j, lane, b.lse);
      stage_dwords(rn, j, lane, b.nd);
    }
  };
  stage_q(0, buf[0]);
  // the lane's key and value: B operands of S = q K^T and dP = dO V^T
  bf16x8 bk[NSUB], bv[NSUB];
#pragma unroll
  for (int c = 0; c < NSUB; ++c) {
    bk[c] = *(const bf16x8*)(Kh + (off + kc) * HD + 32 * c + 8 * g);
    bv[c] = *(const bf16x8*)(Vh + (off + kc) * HD + 32 * c + 8 * g);
  }
  vm_wait(0);
#pragma unroll
  for (int c = 0; c < NSUB; ++c) asm volatile("" : "+v"(bk[c]), "+v"(bv[c]));

  const int qk_off = li * 64 + 16 * (g ^ swz(li));
  const int vr = 4 * g + (li >> 2);
  const int t_off0 = swz_off(vr, 4 * (li & 3)), t_off1 = swz_off(vr, 16 + 4 * (li & 3));
  f32x4 dkacc[HD / 16], dvacc[HD / 16];
#pragma unroll
  for (int d = 0; d < HD / 16; ++d) {
    dkacc[d] = f32x4{};
    dvacc[d] = f32x4{};
  }
  float sat = 0.f;  // the lane's largest clamped |dS| 2^20 (kFixLim once a term saturated)

  for (int qb = 0; qb < nqb; ++qb) {
    vm_wait(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const TiledQBuf<HD>& cur = buf[qb & 1];
    // S - lse = q K^T + bias - lse: lane = key li, rows = queries 16 qt + 4 g + i. The block's
    // LSE and -D and the bias are read before the next block's copies are issued.
    f32x4 lsv[4], ndv[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      lsv[qt] = *(const f32x4*)(cur.lse + 16 * qt + 4 * g);
      ndv[qt] = *(const f32x4*)(cur.nd + 16 * qt + 4 * g);
    }
    // FAST: the pair's clamped table offset (twice its bin, or 2 nbins for masked pairs), which
    // is also its dT bin; otherwise the queries' plain codes
    int cqs[16];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      const int4 cqv = *(const int4*)(cur.codes + 16 * qt + 4 * g);
      const int c4[4] = {cqv.x, cqv.y, cqv.z, cqv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) cqs[4 * qt + i] = FAST ? (int)min((uint32_t)(c4[i] - kenc), lim) : c4[i];
    }
    f32x4 s[4];
    if constexpr (FAST) {
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t raw = *(const unsigned short*)((const char*)sm.tab + cqs[4 * qt + i]);
          s[qt][i] = half_lo_minus(raw, lsv[qt][i]);
        }
    } else {
      float tv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) tv[j] = tab[(cqs[j] & 0xffffff) - (ck & 0xffffff) + code0];
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * qt + i;
          // a padding key and a padding query share the padding label: mask on kv as well
          s[qt][i] = (!kv || (cqs[j] >> 24) != (ck >> 24)) ? -INFINITY : tv[j] * kLog2e - lsv[qt][i];
        }
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) asm volatile("" : "+v"(s[qt]), "+v"(ndv[qt]) : : "memory");
    if (qb + 1 < nqb) stage_q(qb + 1, buf[(qb + 1) & 1]);
    f32x4 p[4], ds[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
#pragma unroll
      for (int c = 0; c < NSUB; ++c) s[qt] = mfma16(*(const bf16x8*)(cur.q[c] + qk_off + 1024 * qt), bk[c], s[qt]);
      f32x4 dp = ndv[qt];
#pragma unroll
      for (int c = 0; c < NSUB; ++c) dp = mfma16(*(const bf16x8*)(cur.d[c] + qk_off + 1024 * qt), bv[c], dp);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[qt][i] = fast_exp2(s[qt][i]);
        ds[qt][i] = p[qt][i] * dp[i];
      }
    }
    // dT: every pair's dS into the workgroup's fixed-point bins
#pragma unroll
    for (int qt = 0; qt < 4; ++qt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float t = fminf(fmaxf(ds[qt][i] * kFix, -kFixLim), kFixLim);  // NaN -> -kFixLim
        sat = fmaxf(sat, fabsf(t));
        const int v = (int)rintf(t);
        if constexpr (FAST) {
          // the clamped offset is even (both encodings are even and the odd padding query code
          // always clamps to 2 nbins), so bin * 8 = offset * 4; masked pairs: bin nbins, v = 0
          lds_add_u64_at(bins_base + ((uint32_t)cqs[4 * qt + i] << 2), (uint64_t)(int64_t)v);
        } else {
          // an allowed pair (v != 0 only then)
          const int bin = (cqs[4 * qt + i] & 0xffffff) - (ck & 0xffffff) + code0;
          if (v != 0) {
            if (global_bins)
              atomicAdd(acc + bin, (unsigned long long)(int64_t)v);
            else
              lds_add_u64(&bins[bin], (uint64_t)(int64_t)v);
          }
        }
      }
    // dV^T += dO^T P and dK^T += q^T dS: B operands are the lane's key column with the
    // queries of two adjacent 16-query tiles
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      bf16x8 pb, db;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = to_bf16(p[2 * cc][i]);
        pb[4 + i] = to_bf16(p[2 * cc + 1][i]);
        db[i] = to_bf16(ds[2 * cc][i]);
        db[4 + i] = to_bf16(ds[2 * cc + 1][i]);
      }
#pragma unroll
      for (int sc = 0; sc < NSUB; ++sc) {
        bf16x8 f0, f1;
        tile_frag_tr2_at(cur.d[sc] + 2048 * cc, t_off0, t_off1, f0, f1);
        dvacc[2 * sc] = mfma16(f0, pb, dvacc[2 * sc]);
        dvacc[2 * sc + 1] = mfma16(f1, pb, dvacc[2 * sc + 1]);
        tile_frag_tr2_at(cur.q[sc] + 2048 * cc, t_off0, t_off1, f0, f1);
        dkacc[2 * sc] = mfma16(f0, db, dkacc[2 * sc]);
        dkacc[2 * sc + 1] = mfma16(f1, db, dkacc[2 * sc + 1]);
      }
    }
  }
  {
    // 16-byte pieces: lanes 16 apart (same key) swap halves (every lane takes part)
    const int64_t grow = kv ? a.perm[off + k] : 0;
    bf16* row = a.dqkv + grow * 3 * a.C + (int64_t)h * HD + pair_col(g);
    const float kscale = 1.f / kLog2e;  // q' = tau log2(e) q
#pragma unroll
    for (int sc = 0; sc < NSUB; ++sc) {
      bf16x4 k0, k1, v0, v1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        k0[i] = to_bf16(dkacc[2 * sc][i] * kscale);
        k1[i] = to_bf16(dkacc[2 * sc + 1][i] * kscale);
        v0[i] = to_bf16(dvacc[2 * sc][i]);
        v1[i] = to_bf16(dvacc[2 * sc + 1][i]);
      }
      const bf16x8 k8 = pair_cols(k0, k1, g), v8 = pair_cols(v0, v1, g);
      if (kv) {
        *(bf16x8*)(row + a.C + 32 * sc) = k8;
        *(bf16x8*)(row + 2 * a.C + 32 * sc) = v8;
      }
    }
  }
  if (sat >= kFixLim) a.dbias_acc[(int64_t)a.nh * a.nbins] = 1ull;  // saturation word (same value from any lane)
  if (global_bins) return;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the bin additions above are inline assembly
  __syncthreads();
  for (int i = threadIdx.x; i < a.nbins; i += 64 * NW) {
    const unsigned long long v = bins[i];
    if (v) atomicAdd(acc + i, v);
  }
}

__global__ __launch_bounds__(256) void k_fixed_zero(unsigned long long* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

// p[n] is the call's saturation word: when set, every entry becomes NaN and the plan's sticky
// flags get SWIN_FLAG_DT_SATURATED.
__global__ __launch_bounds__(256) void k_fixed_to_f32(const unsigned long long* p, float* out, int64_t n,
                                                      unsigned int* flags) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool saturated = p[n] != 0ull;
  if (i < n) out[i] = saturated ? __builtin_nanf("") : (float)((double)(long long)p[i] * (1.0 / kFix));
  if (saturated && i == 0) atomicOr(flags, SWIN_FLAG_DT_SATURATED);
}

static TiledArgs tiled_args(const swin_attn_plan* p) {
  TiledArgs a{};
  a.perm = p->dev.perm;
  a.work = p->dev.tiled_work;
  a.kv_work = p->dev.tiled_kv_work;
  a.codes = p->dev.tiled_codes;
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
  // 4 waves of 32 queries: blocks of 128 queries (the 128-token work items), two workgroups per CU
  const bool fast = p->nbins <= kTabLds;
  a.work = p->dev.tiled_kv_work;
  const dim3 grid((unsigned)p->tiled_kv_work.size(), (unsigned)p->nh);
  if (p->hd == 32)
    fast ? k_tiled_fwd_pipe<32, true><<<grid, 256, 0, s>>>(a) : k_tiled_fwd_pipe<32, false><<<grid, 256, 0, s>>>(a);
  else if (p->hd == 64)
    fast ? k_tiled_fwd_pipe<64, true><<<grid, 256, 0, s>>>(a) : k_tiled_fwd_pipe<64, false><<<grid, 256, 0, s>>>(a);
  else
    fast ? k_tiled_fwd_pipe<128, true><<<grid, 256, 0, s>>>(a) : k_tiled_fwd_pipe<128, false><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int HD>
static hipError_t tiled_bwd_launch(const TiledArgs& a, unsigned items, unsigned kv_items, int nh, hipStream_t s) {
  if (a.nbins <= kTabLds)
    k_tiled_bwd_dkv<HD, true><<<dim3(kv_items, (unsigned)nh), 64 * kKvWaves, 0, s>>>(a);
  else
    k_tiled_bwd_dkv<HD, false><<<dim3(kv_items, (unsigned)nh), 64 * kKvWaves, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.nbins <= kTabLds)
    k_tiled_bwd_dq<HD, true><<<dim3(items, (unsigned)nh), 256, 0, s>>>(a);
  else
    k_tiled_bwd_dq<HD, false><<<dim3(items, (unsigned)nh), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_tiled_bwd_bf16(const swin_attn_plan* p, const void* qkv, const float* lse, const void* dO,
                                 const float* dd, const float* table, void* dqkv, unsigned long long* acc,
                                 float* dtable, hipStream_t s) {
  TiledArgs a = tiled_args(p);
  a.qkv = (const bf16*)qkv;
  a.lse = (float*)lse;
  a.dO = (const bf16*)dO;
  a.dd = dd;
  a.table = table;
  a.dqkv = (bf16*)dqkv;
  a.dbias_acc = acc;
  const int64_t nacc = (int64_t)p->nh * p->nbins;
  k_fixed_zero<<<(unsigned)((nacc + 1 + 255) / 256), 256, 0, s>>>(acc, nacc + 1);  // and the saturation word
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned items = (unsigned)p->tiled_work.size(), kv_items = (unsigned)p->tiled_kv_work.size();
  if (p->hd == 32)
    e = tiled_bwd_launch<32>(a, items, kv_items, p->nh, s);
  else if (p->hd == 64)
    e = tiled_bwd_launch<64>(a, items, kv_items, p->nh, s);
  else
    e = tiled_bwd_launch<128>(a, items, kv_items, p->nh, s);
  if (e != hipSuccess) return e;
  k_fixed_to_f32<<<(unsigned)((nacc + 255) / 256), 256, 0, s>>>(acc, dtable, nacc, p->dev.flags);
  return hipGetLastError();
}

}  // namespace swin
