// fp32 forward path: the same module as the bf16 path (QKV projection with the cyclic
// shift + window partition fused into its operand load, window attention with the
// relative-position bias and shift mask, projection with the window reverse + un-shift
// fused into its store), computed in fp32 on the vector ALUs. It serves the fp32
// configurations, whose size is small; the bf16 path is the fast one.
#include <math.h>

#include "device_common.h"
#include "swin_internal.h"

namespace swin {

// C[m, n] = sum_k A[row(m), k] * B[n, k] + bias[n]. mode 1 writes head-split planes
// [3][nh][n_tok][hd]; mode 0 writes rows, optionally scattered through out_rows.
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ A, const int32_t* __restrict__ a_rows,
                                                  const float* __restrict__ B, const float* __restrict__ bias,
                                                  int64_t M, int N, int K, int mode, float* __restrict__ out,
                                                  const int32_t* __restrict__ out_rows, int C, int nh, int hd,
                                                  int64_t n_tok) {
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[16][64 + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 64;
  const int n0 = blockIdx.y * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int i = threadIdx.x; i < 64 * 16; i += 256) {
      const int r = i / 16, kk = i % 16;
      const int64_t m = m0 + r;
      const int n = n0 + r;
      float av = 0.f, bv = 0.f;
      if (m < M && k0 + kk < K) av = A[(a_rows ? (int64_t)a_rows[m] : m) * K + k0 + kk];
      if (n < N && k0 + kk < K) bv = B[(int64_t)n * K + k0 + kk];
      As[kk][r] = av;
      Bs[kk][r] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(As[kk][ty * 4 + i], Bs[kk][tx * 4 + j], acc[i][j]);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      const float v = acc[i][j] + (bias ? bias[n] : 0.f);
      if (mode == 1) {
        const int plane = n / C, rem = n % C, head = rem / hd, d = rem % hd;
        out[(((int64_t)plane * nh + head) * n_tok + m) * hd + d] = v;
      } else {
        out[(out_rows ? (int64_t)out_rows[m] : m) * N + n] = v;
      }
    }
  }
}

// One workgroup per (window, head); one thread per query with an online softmax over the
// window's keys (K and V staged in LDS). HDM bounds head_dim (32 or 64): the per-query
// vectors are unrolled over HDM with a head_dim guard, so they live in registers. The bias
// table index of a pair is linear in the two tokens' window coordinates, bin = qpos - kpos +
// const, so each key's kpos and wrap label are formed once per workgroup in LDS. EXACT:
// head_dim equals HDM (no guards).
template <int HDM, bool EXACT>
__global__ __launch_bounds__(256) void k_attn_f32(const float* __restrict__ qkv, const float* __restrict__ table,
                                                  float* __restrict__ o, float* __restrict__ lse,
                                                  const ClassInfo* __restrict__ classes,
                                                  const int32_t* __restrict__ class_win,
                                                  const int32_t* __restrict__ win_off, int64_t n_tok, int nh, int C,
                                                  int hd_arg, int nbins, int wd, int wh, int ww, float tau,
                                                  int n_cls) {
  extern __shared__ float sm[];
  const int hd = EXACT ? HDM : hd_arg;
  const int h = blockIdx.y;
  const int slot = blockIdx.x;  // index into the class-sorted window list
  int c = 0;
  while (c + 1 < n_cls && classes[c + 1].first <= slot) ++c;
  const ClassInfo ci = classes[c];
  const int n = ci.n;
  const int64_t off = win_off[class_win[slot]];
  float* Ks = sm;
  float* Vs = sm + n * hd;
  int2* kinfo = (int2*)(Vs + n * hd);  // per key: (position term of the bin, wrap label)
  const float* Qh = qkv + ((int64_t)(0 * nh + h) * n_tok + off) * hd;
  const float* Kh = qkv + ((int64_t)(1 * nh + h) * n_tok + off) * hd;
  const float* Vh = qkv + ((int64_t)(2 * nh + h) * n_tok + off) * hd;
  for (int i = threadIdx.x; i < n * hd; i += blockDim.x) {
    Ks[i] = Kh[i];
    Vs[i] = Vh[i];
  }
  const int th = 2 * wh - 1, tw = 2 * ww - 1;
  auto coords = [&](int t, int& pos, int& lab) {
    const int tw_ = t % ci.ext[2], th_ = (t / ci.ext[2]) % ci.ext[1], td_ = t / (ci.ext[2] * ci.ext[1]);
    pos = (td_ * th + th_) * tw + tw_;
    lab = (td_ >= ci.split[0]) | ((th_ >= ci.split[1]) << 1) | ((tw_ >= ci.split[2]) << 2);
  };
  for (int k = threadIdx.x; k < n; k += blockDim.x) {
    int pos, lab;
    coords(k, pos, lab);
    kinfo[k] = int2{pos, lab};
  }
  __syncthreads();
  const float* tab = table + (int64_t)h * nbins;
  const int bin0 = ((wd - 1) * th + (wh - 1)) * tw + (ww - 1);  // bin of a pair at zero offset
  for (int q = threadIdx.x; q < n; q += blockDim.x) {
    float qv[HDM], acc[HDM];
#pragma unroll
    for (int d = 0; d < HDM; ++d) {
      qv[d] = d < hd ? Qh[(int64_t)q * hd + d] * tau : 0.f;
      acc[d] = 0.f;
    }
    int qpos, ql;
    coords(q, qpos, ql);
    const float* tq = tab + bin0 + qpos;  // tq[-kpos] is the pair's bias
    float m = -INFINITY, l = 0.f;
    for (int k = 0; k < n; ++k) {
      const int2 ki = kinfo[k];
      if (ki.y != ql) continue;
      const float* kr = Ks + k * hd;
      const float* vr = Vs + k * hd;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < HDM; ++d)
        if (d < hd) s = fmaf(qv[d], kr[d], s);
      s += tq[-ki.x];
      const float mn = fmaxf(m, s);
      const float corr = expf(m - mn);
      const float p = expf(s - mn);
      l = l * corr + p;
#pragma unroll
      for (int d = 0; d < HDM; ++d)
        if (d < hd) acc[d] = acc[d] * corr + p * vr[d];
      m = mn;
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < HDM; ++d)
      if (d < hd) o[(off + q) * C + h * hd + d] = acc[d] * inv;
    lse[(int64_t)h * n_tok + off + q] = m + logf(l);
  }
}

hipError_t launch_fwd_f32(const swin_attn_plan* p, const void* x, const void* w_qkv, const void* b_qkv,
                          const void* w_proj, const void* b_proj, const float* table, void* y, void* saved,
                          hipStream_t s) {
  char* base = (char*)saved;
  float* qkv = (float*)base;
  float* o = (float*)(base + p->saved_qkv);
  float* lse = (float*)(base + p->saved_qkv + p->saved_o);
  const int C = p->C;
  dim3 g1((unsigned)((p->n_tok + 63) / 64), (unsigned)((3 * C + 63) / 64));
  k_gemm_f32<<<g1, 256, 0, s>>>((const float*)x, p->dev.perm, (const float*)w_qkv, (const float*)b_qkv, p->n_tok,
                                3 * C, C, 1, qkv, nullptr, C, p->nh, p->hd, p->n_tok);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = 2 * (size_t)p->stats.max_tokens * p->hd * sizeof(float) + (size_t)p->stats.max_tokens * 8;
  const dim3 ga((unsigned)p->n_win, (unsigned)p->nh);
  auto attn = [&](auto kern) {
    kern<<<ga, 256, lds, s>>>(qkv, table, o, lse, p->dev.classes, p->dev.class_win, p->dev.win_off, p->n_tok, p->nh,
                              C, p->hd, p->nbins, p->d.window[0], p->d.window[1], p->d.window[2], p->tau,
                              (int)p->classes.size());
  };
  if (p->hd == 32)
    attn(k_attn_f32<32, true>);
  else if (p->hd == 64)
    attn(k_attn_f32<64, true>);
  else if (p->hd < 32)
    attn(k_attn_f32<32, false>);
  else
    attn(k_attn_f32<64, false>);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2((unsigned)((p->n_tok + 63) / 64), (unsigned)((C + 63) / 64));
  k_gemm_f32<<<g2, 256, 0, s>>>(o, nullptr, (const float*)w_proj, (const float*)b_proj, p->n_tok, C, C, 0,
                                (float*)y, p->dev.perm, C, p->nh, p->hd, p->n_tok);
  return hipGetLastError();
}

}  // namespace swin
