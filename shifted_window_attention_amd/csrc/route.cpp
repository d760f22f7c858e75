// Token routes between rank layouts (include/swin_route.h): host planning of the per-rank
// index tables, and the pack / loopback exchange / restore launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "../../include/swin_route.h"
#include "swin_internal.h"

namespace {

swin_status fail(swin_status st, const std::string& msg) {
  swin::set_error(msg);
  return st;
}

swin_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SWIN_OK;
  swin::set_error(std::string(what) + ": " + hipGetErrorString(e));
  return SWIN_ERR_HIP;
}

// Eq. 4 split of n items over k ranks: rank i gets [floor(i n / k), floor((i + 1) n / k)).
int64_t eq4_lo(int64_t n, int64_t k, int64_t i) { return (i * n) / k; }

// Where every token (flat grid index) lives in one layout.
struct Placement {
  int ranks = 0;
  std::vector<int32_t> rank, off;       // per token
  std::vector<int64_t> size;            // per rank
  std::vector<std::vector<int32_t>> by_off;  // per rank: token at each local offset
};

swin_status place(const swin_attn_desc& g, const swin_rank_layout& L, Placement& P) {
  const int64_t B = g.batch, D = g.grid[0], H = g.grid[1], W = g.grid[2];
  const int64_t n = B * D * H * W;
  if (L.ranks < 1) return fail(SWIN_ERR_ARG, "a layout needs ranks >= 1");
  P.ranks = L.ranks;
  P.rank.assign(n, -1);
  P.off.assign(n, -1);
  P.size.assign(L.ranks, 0);
  P.by_off.assign(L.ranks, {});
  if (L.kind == SWIN_LAYOUT_STRIPES) {
    if (L.shift[0] || L.shift[1] || L.shift[2]) return fail(SWIN_ERR_ARG, "a stripe layout has no shift");
    if (L.ranks > H) return fail(SWIN_ERR_ARG, "more stripes than latitude rows");
    std::vector<int32_t> row_rank(H);
    std::vector<int64_t> lo(L.ranks + 1);
    for (int p = 0; p <= L.ranks; ++p) lo[p] = eq4_lo(H, L.ranks, p);
    for (int p = 0; p < L.ranks; ++p)
      for (int64_t h = lo[p]; h < lo[p + 1]; ++h) row_rank[h] = p;
    for (int p = 0; p < L.ranks; ++p) {
      P.size[p] = B * D * (lo[p + 1] - lo[p]) * W;
      P.by_off[p].resize(P.size[p]);
    }
    for (int64_t b = 0; b < B; ++b)
      for (int64_t d = 0; d < D; ++d)
        for (int64_t h = 0; h < H; ++h) {
          const int p = row_rank[h];
          const int64_t rows = lo[p + 1] - lo[p];
          for (int64_t w = 0; w < W; ++w) {
            const int64_t tok = ((b * D + d) * H + h) * W + w;
            const int64_t o = ((b * D + d) * rows + (h - lo[p])) * W + w;
            P.rank[tok] = p;
            P.off[tok] = (int32_t)o;
            P.by_off[p][o] = (int32_t)tok;
          }
        }
    return SWIN_OK;
  }
  if (L.kind != SWIN_LAYOUT_WINDOWS) return fail(SWIN_ERR_ARG, "unknown layout kind");
  swin_attn_desc d = g;
  d.heads = 1;
  d.scale = 0.f;
  for (int a = 0; a < 3; ++a) d.shift[a] = L.shift[a];
  std::vector<int64_t> perm(n);
  swin_status st = swin_attn_host_index_map(&d, perm.data(), nullptr);
  if (st != SWIN_OK) return st;
  // window starts in the module's row-major window order (the index map's slot order)
  std::vector<int64_t> start;
  int64_t nk[3];
  for (int a = 0; a < 3; ++a) nk[a] = (d.grid[a] + d.window[a] - 1) / d.window[a];
  int64_t slot = 0;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t kd = 0; kd < nk[0]; ++kd)
      for (int64_t kh = 0; kh < nk[1]; ++kh)
        for (int64_t kw = 0; kw < nk[2]; ++kw) {
          start.push_back(slot);
          const int64_t k[3] = {kd, kh, kw};
          int64_t cnt = 1;
          for (int a = 0; a < 3; ++a) cnt *= std::min<int64_t>(d.window[a], d.grid[a] - k[a] * d.window[a]);
          slot += cnt;
        }
  start.push_back(slot);
  const int64_t M = (int64_t)start.size() - 1;
  for (int r = 0; r < L.ranks; ++r) {
    const int64_t s0 = start[eq4_lo(M, L.ranks, r)], s1 = start[eq4_lo(M, L.ranks, r + 1)];
    P.size[r] = s1 - s0;
    P.by_off[r].resize(s1 - s0);
    for (int64_t s = s0; s < s1; ++s) {
      const int64_t tok = perm[s];
      P.rank[tok] = r;
      P.off[tok] = (int32_t)(s - s0);
      P.by_off[r][s - s0] = (int32_t)tok;
    }
  }
  return SWIN_OK;
}

struct HostRoute {
  int P = 0, R = 0;
  int64_t n = 0;
  std::vector<int64_t> counts;                 // [P][R]
  std::vector<int64_t> src_size, dst_size;
  std::vector<int32_t> send_src, recv_dst;     // concatenated over ranks
  std::vector<int64_t> src_base, dst_base;     // first row of each rank in the concatenations
};

// The route uses the descriptor's ndim, dtype, batch, grid, channels, window and periodic
// fields; heads, shift and scale are ignored, so they are neutralised before validation.
swin_status validate_grid(const swin_attn_desc* g) {
  if (!g) return fail(SWIN_ERR_ARG, "grid descriptor is NULL");
  swin_attn_desc d = *g;
  d.shift[0] = d.shift[1] = d.shift[2] = 0;
  d.heads = 1;
  d.scale = 0.f;
  swin_attn_stats st{};
  return swin_attn_host_stats(&d, &st);  // validates grid, window, dtype, channels, sizes
}

swin_status build_route(const swin_attn_desc* g, const swin_rank_layout* src, const swin_rank_layout* dst,
                        HostRoute& H) {
  if (!src || !dst) return fail(SWIN_ERR_ARG, "NULL layout");
  swin_status st = validate_grid(g);
  if (st != SWIN_OK) return st;
  Placement S, T;
  st = place(*g, *src, S);
  if (st == SWIN_OK) st = place(*g, *dst, T);
  if (st != SWIN_OK) return st;
  H.P = S.ranks;
  H.R = T.ranks;
  H.n = (int64_t)S.rank.size();
  H.counts.assign((size_t)H.P * H.R, 0);
  H.src_size = S.size;
  H.dst_size = T.size;
  // segments (p -> r), each in destination-offset order: walk every destination's rows in order
  std::vector<std::vector<int32_t>> seg_src((size_t)H.P * H.R), seg_dst((size_t)H.P * H.R);
  for (int r = 0; r < H.R; ++r)
    for (int64_t o = 0; o < T.size[r]; ++o) {
      const int32_t tok = T.by_off[r][o];
      const int p = S.rank[tok];
      seg_src[(size_t)p * H.R + r].push_back(S.off[tok]);
      seg_dst[(size_t)p * H.R + r].push_back((int32_t)o);
    }
  H.send_src.reserve(H.n);
  H.recv_dst.reserve(H.n);
  H.src_base.assign(H.P + 1, 0);
  H.dst_base.assign(H.R + 1, 0);
  for (int p = 0; p < H.P; ++p) {
    H.src_base[p] = (int64_t)H.send_src.size();
    for (int r = 0; r < H.R; ++r) {
      const auto& v = seg_src[(size_t)p * H.R + r];
      H.counts[(size_t)p * H.R + r] = (int64_t)v.size();
      H.send_src.insert(H.send_src.end(), v.begin(), v.end());
    }
  }
  H.src_base[H.P] = (int64_t)H.send_src.size();
  for (int r = 0; r < H.R; ++r) {
    H.dst_base[r] = (int64_t)H.recv_dst.size();
    for (int p = 0; p < H.P; ++p) {
      const auto& v = seg_dst[(size_t)p * H.R + r];
      H.recv_dst.insert(H.recv_dst.end(), v.begin(), v.end());
    }
  }
  H.dst_base[H.R] = (int64_t)H.recv_dst.size();
  return SWIN_OK;
}

}  // namespace

struct swin_route_plan {
  HostRoute h;
  size_t row_bytes = 0;
  int32_t* d_send_src = nullptr;
  int32_t* d_recv_dst = nullptr;
};

extern "C" {

swin_status swin_route_host_tables(const swin_attn_desc* grid, const swin_rank_layout* src,
                                   const swin_rank_layout* dst, int64_t* counts, int32_t* send_src,
                                   int32_t* recv_dst) {
  HostRoute h;
  swin_status st = build_route(grid, src, dst, h);
  if (st != SWIN_OK) return st;
  if (counts) std::copy(h.counts.begin(), h.counts.end(), counts);
  if (send_src) std::copy(h.send_src.begin(), h.send_src.end(), send_src);
  if (recv_dst) std::copy(h.recv_dst.begin(), h.recv_dst.end(), recv_dst);
  return SWIN_OK;
}

swin_status swin_route_plan_create(const swin_attn_desc* grid, const swin_rank_layout* src,
                                   const swin_rank_layout* dst, swin_route_plan** out) {
  if (!out) return fail(SWIN_ERR_ARG, "plan output is NULL");
  *out = nullptr;
  swin_route_plan* p = new (std::nothrow) swin_route_plan();
  if (!p) return fail(SWIN_ERR_ARG, "out of host memory");
  swin_status st = build_route(grid, src, dst, p->h);
  if (st != SWIN_OK) {
    delete p;
    return st;
  }
  p->row_bytes = (size_t)grid->channels * (grid->dtype == SWIN_BF16 ? 2 : 4);
  const size_t bytes = (size_t)std::max<int64_t>(p->h.n, 1) * 4;
  hipError_t e = hipMalloc(&p->d_send_src, bytes);
  if (e == hipSuccess) e = hipMalloc(&p->d_recv_dst, bytes);
  if (e == hipSuccess && p->h.n)
    e = hipMemcpy(p->d_send_src, p->h.send_src.data(), p->h.n * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess && p->h.n)
    e = hipMemcpy(p->d_recv_dst, p->h.recv_dst.data(), p->h.n * 4, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    swin_route_plan_destroy(p);
    return hip_status(e, "route table upload");
  }
  *out = p;
  return SWIN_OK;
}

void swin_route_plan_destroy(swin_route_plan* plan) {
  if (!plan) return;
  if (plan->d_send_src) (void)hipFree(plan->d_send_src);
  if (plan->d_recv_dst) (void)hipFree(plan->d_recv_dst);
  delete plan;
}

swin_status swin_route_counts(const swin_route_plan* plan, int64_t* counts, int64_t* src_sizes, int64_t* dst_sizes) {
  if (!plan) return fail(SWIN_ERR_ARG, "plan is NULL");
  if (counts) std::copy(plan->h.counts.begin(), plan->h.counts.end(), counts);
  if (src_sizes) std::copy(plan->h.src_size.begin(), plan->h.src_size.end(), src_sizes);
  if (dst_sizes) std::copy(plan->h.dst_size.begin(), plan->h.dst_size.end(), dst_sizes);
  return SWIN_OK;
}

swin_status swin_route_pack(const swin_route_plan* plan, int32_t p, const void* local, void* send, void* stream) {
  if (!plan) return fail(SWIN_ERR_ARG, "plan is NULL");
  if (p < 0 || p >= plan->h.P) return fail(SWIN_ERR_ARG, "source rank out of range");
  const int64_t n = plan->h.src_size[p];
  if (n == 0) return SWIN_OK;
  if (!local || !send) return fail(SWIN_ERR_ARG, "NULL buffer");
  if (local == send) return fail(SWIN_ERR_ARG, "send must not alias local");
  return hip_status(swin::launch_rows_move(local, send, plan->d_send_src + plan->h.src_base[p], n, plan->row_bytes,
                                           false, (hipStream_t)stream),
                    "route pack");
}

swin_status swin_route_unpack(const swin_route_plan* plan, int32_t r, const void* recv, void* local, void* stream) {
  if (!plan) return fail(SWIN_ERR_ARG, "plan is NULL");
  if (r < 0 || r >= plan->h.R) return fail(SWIN_ERR_ARG, "destination rank out of range");
  const int64_t n = plan->h.dst_size[r];
  if (n == 0) return SWIN_OK;
  if (!local || !recv) return fail(SWIN_ERR_ARG, "NULL buffer");
  if (local == recv) return fail(SWIN_ERR_ARG, "local must not alias recv");
  return hip_status(swin::launch_rows_move(recv, local, plan->d_recv_dst + plan->h.dst_base[r], n, plan->row_bytes,
                                           true, (hipStream_t)stream),
                    "route unpack");
}

swin_status swin_route_loopback(const swin_route_plan* plan, const void* const* send, void* const* recv, void* stream) {
  if (!plan) return fail(SWIN_ERR_ARG, "plan is NULL");
  if (!send || !recv) return fail(SWIN_ERR_ARG, "NULL buffer arrays");
  const HostRoute& h = plan->h;
  for (int p = 0; p < h.P; ++p)
    if (h.src_size[p] && !send[p]) return fail(SWIN_ERR_ARG, "NULL send buffer of a rank with tokens");
  for (int r = 0; r < h.R; ++r)
    if (h.dst_size[r] && !recv[r]) return fail(SWIN_ERR_ARG, "NULL receive buffer of a rank with tokens");
  // segment (p -> r) starts after the segments (p -> r' < r) in send[p] and (p' < p -> r) in recv[r]
  std::vector<int64_t> recv_pos(h.R, 0);
  for (int p = 0; p < h.P; ++p) {
    int64_t send_pos = 0;
    for (int r = 0; r < h.R; ++r) {
      const int64_t c = h.counts[(size_t)p * h.R + r];
      if (c) {
        const hipError_t e =
            hipMemcpyAsync((char*)recv[r] + recv_pos[r] * plan->row_bytes,
                           (const char*)send[p] + send_pos * plan->row_bytes, c * plan->row_bytes,
                           hipMemcpyDeviceToDevice, (hipStream_t)stream);
        if (e != hipSuccess) return hip_status(e, "route loopback copy");
      }
      send_pos += c;
      recv_pos[r] += c;
    }
  }
  return SWIN_OK;
}

}  // extern "C"
