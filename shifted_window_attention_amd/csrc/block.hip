// Swin Transformer block around the attention module (TERRA section IV-A, Fig. 4: block 0
// is W-MSA followed by an MLP, block 1 SW-MSA followed by an MLP, with layer
// normalisation), read as the pre-normalisation block
//     h = x + A(LN1(x)),        y = h + W2 GELU(W1 LN2(h) + b1) + b2.
//
// Layer normalisation has kernels of its own (one wave per token row, fp32 statistics);
// the residual adds, the MLP bias + GELU and the GELU derivative are fused into the
// epilogues of the row GEMMs, and the MLP weight gradients use the split-K token
// contraction of the attention module.
#include "device_common.h"
#include "swin_internal.h"

namespace swin {

__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// Eight consecutive channels of a bf16 or fp32 row as fp32 (one 16-byte load, or two).
__device__ __forceinline__ void load8(const bf16* p, float (&v)[8]) {
  const bf16x8 t = *(const bf16x8*)p;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = to_f32(t[e]);
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = a[e];
    v[4 + e] = b[e];
  }
}

// y = (x - mean) rstd g + b per row of C channels (biased variance, fp32 statistics);
// mean and rstd are saved for the backward. One wave per row, lane l holds the 8-channel
// chunks l, l + 64, ... (CH of them).
template <int CH, typename TX>
__global__ __launch_bounds__(256) void k_layernorm_fwd(const TX* __restrict__ x, const bf16* __restrict__ g,
                                                       const bf16* __restrict__ b, bf16* __restrict__ y,
                                                       float* __restrict__ mean_out, float* __restrict__ rstd_out,
                                                       int64_t rows, int C, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nch = C / 8;
  float v[CH][8];
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch) {
      load8(x + row * C + 8 * ch, v[c]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[c][e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sum += v[c][e];
  }
  const float mean = wave_sum64(sum) / C;
  float sq = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
    if (lane + 64 * c < nch)
#pragma unroll
      for (int e = 0; e < 8; ++e) sq += (v[c][e] - mean) * (v[c][e] - mean);
  const float rstd = rsqrtf(wave_sum64(sq) / C + eps);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch) {
      const bf16x8 gg = *(const bf16x8*)(g + 8 * ch), bb = *(const bf16x8*)(b + 8 * ch);
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = to_bf16((v[c][e] - mean) * rstd * to_f32(gg[e]) + to_f32(bb[e]));
      *(bf16x8*)(y + row * C + 8 * ch) = o;
    }
  }
  if (lane == 0) {
    mean_out[row] = mean;
    rstd_out[row] = rstd;
  }
}

// Backward of k_layernorm_fwd (upstream gradient dy in fp32: the products that produce it write
// fp32) plus a residual gradient:
//   dx = dres + rstd (dxhat - mean(dxhat) - xhat mean(dxhat xhat)),  dxhat = dy g,
// rounded once to bf16 (and also stored in fp32 when dx32 is given: the block's residual
// gradient stream stays in fp32),
// and, per workgroup (a contiguous range of `per` rows), partial sums of dg = sum dy xhat
// and db = sum dy (part[group][0][:] and part[group][1][:]), combined over the 4 waves in a
// fixed order. At most kLnMaxGroups workgroups, so that the final reduction stays short.
template <int CH, typename TX, typename TR>
__global__ __launch_bounds__(256) void k_layernorm_bwd(const float* __restrict__ dy, const TX* __restrict__ x,
                                                       const float* __restrict__ mean, const float* __restrict__ rstd,
                                                       const bf16* __restrict__ g, const TR* __restrict__ dres,
                                                       bf16* __restrict__ dx, float* __restrict__ dx32,
                                                       float* __restrict__ part, int64_t rows, int64_t per, int C) {
  __shared__ float red[4][2][64 * 8 * CH];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nch = C / 8;
  const int64_t r0 = (int64_t)blockIdx.x * per;
  const int64_t r1 = r0 + per < rows ? r0 + per : rows;
  float gv[CH][8], dg[CH][8], db[CH][8];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = lane + 64 * c;
    const bf16x8 t = ch < nch ? *(const bf16x8*)(g + 8 * ch) : bf16x8{};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      gv[c][e] = to_f32(t[e]);
      dg[c][e] = 0.f;
      db[c][e] = 0.f;
    }
  }
  for (int64_t row = r0 + w; row < r1; row += 4) {
    const float mu = mean[row], rs = rstd[row];
    float xh[CH][8], dxh[CH][8];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ch = lane + 64 * c;
      float tx[8];
      if (ch < nch) {
        load8(x + row * C + 8 * ch, tx);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) tx[e] = 0.f;
      }
      float ty[8];
      if (ch < nch) {
        load8(dy + row * C + 8 * ch, ty);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) ty[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = ty[e];
        xh[c][e] = ch < nch ? (tx[e] - mu) * rs : 0.f;
        dxh[c][e] = d * gv[c][e];
        s1 += dxh[c][e];
        s2 += dxh[c][e] * xh[c][e];
        dg[c][e] += d * xh[c][e];
        db[c][e] += d;
      }
    }
    s1 = wave_sum64(s1) / C;
    s2 = wave_sum64(s2) / C;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nch) {
        float tr[8], r[8];
        load8(dres + row * C + 8 * ch, tr);
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          r[e] = rs * (dxh[c][e] - s1 - xh[c][e] * s2) + tr[e];
          o[e] = to_bf16(r[e]);
        }
        *(bf16x8*)(dx + row * C + 8 * ch) = o;
        if (dx32) {
          float* d32 = dx32 + row * C + 8 * ch;
          *(f32x4*)d32 = f32x4{r[0], r[1], r[2], r[3]};
          *(f32x4*)(d32 + 4) = f32x4{r[4], r[5], r[6], r[7]};
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      red[w][0][8 * (lane + 64 * c) + e] = dg[c][e];
      red[w][1][8 * (lane + 64 * c) + e] = db[c][e];
    }
  __syncthreads();
  float* out = part + (int64_t)blockIdx.x * 2 * C;
  for (int i = threadIdx.x; i < 2 * C; i += 256) {
    const int k = i / C, c = i - k * C;
    out[i] = ((red[0][k][c] + red[1][k][c]) + red[2][k][c]) + red[3][k][c];
  }
}

// out[i] = sum over groups of part[g][i], i < n, in a fixed order: each of 4 waves sums the
// groups congruent to its index mod 4 (ascending), then the 4 sums are added in wave order.
// The first half of the n outputs goes to dg, the second to db. One workgroup per 64 outputs.
__global__ __launch_bounds__(256) void k_reduce_groups(const float* __restrict__ part, int groups, int n,
                                                       float* __restrict__ dg, float* __restrict__ db) {
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + lane;
  float acc = 0.f;
  if (i < n) {
#pragma unroll 8
    for (int k = q; k < groups; k += 4) acc += part[(int64_t)k * n + i];
  }
  red[q][lane] = acc;
  __syncthreads();
  if (q == 0 && i < n) {
    const float v = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
    const int C = n / 2;
    if (i < C)
      dg[i] = v;
    else
      db[i - C] = v;
  }
}

template <typename TX>
hipError_t launch_layernorm_fwd(const TX* x, const bf16* g, const bf16* b, bf16* y, float* mean, float* rstd,
                                int64_t rows, int C, float eps, hipStream_t s) {
  const unsigned blocks = (unsigned)((rows + 3) / 4);
  if (C <= 512)
    k_layernorm_fwd<1, TX><<<blocks, 256, 0, s>>>(x, g, b, y, mean, rstd, rows, C, eps);
  else
    k_layernorm_fwd<2, TX><<<blocks, 256, 0, s>>>(x, g, b, y, mean, rstd, rows, C, eps);
  return hipGetLastError();
}
template hipError_t launch_layernorm_fwd<bf16>(const bf16*, const bf16*, const bf16*, bf16*, float*, float*, int64_t,
                                               int, float, hipStream_t);
template hipError_t launch_layernorm_fwd<float>(const float*, const bf16*, const bf16*, bf16*, float*, float*, int64_t,
                                                int, float, hipStream_t);

template <typename TX, typename TR>
hipError_t launch_layernorm_bwd(const float* dy, const TX* x, const float* mean, const float* rstd, const bf16* g,
                                const TR* dres, bf16* dx, float* dx32, float* part, float* dg, float* db, int64_t rows,
                                int C, hipStream_t s) {
  const int groups = layernorm_groups(rows);
  const int64_t per = ln_rows_per_group(rows);
  if (C <= 512)
    k_layernorm_bwd<1, TX, TR><<<groups, 256, 0, s>>>(dy, x, mean, rstd, g, dres, dx, dx32, part, rows, per, C);
  else
    k_layernorm_bwd<2, TX, TR><<<groups, 256, 0, s>>>(dy, x, mean, rstd, g, dres, dx, dx32, part, rows, per, C);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_reduce_groups<<<(unsigned)((2 * C + 63) / 64), 256, 0, s>>>(part, groups, 2 * C, dg, db);
  return hipGetLastError();
}
// LN2 of the block: fp32 h, bf16 dy; LN1: bf16 x, fp32 residual gradient
template hipError_t launch_layernorm_bwd<float, bf16>(const float*, const float*, const float*, const float*,
                                                      const bf16*, const bf16*, bf16*, float*, float*, float*, float*,
                                                      int64_t, int, hipStream_t);
template hipError_t launch_layernorm_bwd<bf16, float>(const float*, const bf16*, const float*, const float*,
                                                      const bf16*, const float*, bf16*, float*, float*, float*, float*,
                                                      int64_t, int, hipStream_t);

}  // namespace swin
