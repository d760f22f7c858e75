// Host plan and C ABI of the shifted-window attention library.
//
// The plan turns a descriptor into the tables the kernels run from:
//   * the window-major slot -> grid row map (roll by -shift, row-major window
//     order, row-major tokens inside a window; TERRA section IV-D and V-A),
//   * the per-window token offset/length table, which lets short edge windows
//     run without padding,
//   * window classes (extent + wrap-label split) and per-class work chunks.
#include <functional>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <new>
#include <string>
#include <tuple>
#include <vector>

#include "swin_internal.h"

namespace swin {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

struct TraceState {
  void* const* events = nullptr;
  int capacity = 0;
  int cursor = 0;
};
static thread_local TraceState g_trace;

hipError_t trace_mark(hipStream_t s) {
  if (!g_trace.events || g_trace.cursor >= g_trace.capacity) return hipSuccess;
  return hipEventRecord((hipEvent_t)g_trace.events[g_trace.cursor++], s);
}

static swin_status fail(swin_status st, const std::string& msg) {
  set_error(msg);
  return st;
}

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Validate a descriptor; fills a short reason on failure.
static swin_status validate(const swin_attn_desc* d) {
  if (!d) return fail(SWIN_ERR_ARG, "descriptor is NULL");
  if (d->ndim != 2 && d->ndim != 3) return fail(SWIN_ERR_ARG, "ndim must be 2 or 3");
  if (d->dtype != SWIN_F32 && d->dtype != SWIN_BF16) return fail(SWIN_ERR_ARG, "dtype must be SWIN_F32 or SWIN_BF16");
  if (d->batch < 1) return fail(SWIN_ERR_ARG, "batch must be >= 1");
  for (int a = 0; a < 3; ++a) {
    if (d->grid[a] < 1) return fail(SWIN_ERR_ARG, "grid extents must be >= 1");
    if (d->window[a] < 1) return fail(SWIN_ERR_ARG, "window extents must be >= 1");
    if (d->window[a] > d->grid[a]) return fail(SWIN_ERR_ARG, "window larger than the grid");
    if (d->shift[a] < 0 || d->shift[a] >= d->window[a]) return fail(SWIN_ERR_ARG, "shift must satisfy 0 <= s < window");
  }
  if (d->ndim == 2 && (d->grid[0] != 1 || d->window[0] != 1 || d->shift[0] != 0))
    return fail(SWIN_ERR_ARG, "2-D descriptors need grid[0] == window[0] == 1 and shift[0] == 0");
  if (d->channels < 1 || d->heads < 1) return fail(SWIN_ERR_ARG, "channels and heads must be >= 1");
  if (d->channels % d->heads != 0) return fail(SWIN_ERR_ARG, "channels must be a multiple of heads");
  if (d->periodic > 7u) return fail(SWIN_ERR_ARG, "periodic has bits outside 0x7");
  if (!(d->scale >= 0.f) || !std::isfinite(d->scale)) return fail(SWIN_ERR_ARG, "scale must be finite and >= 0");
  const double ntok = double(d->batch) * double(d->grid[0]) * double(d->grid[1]) * double(d->grid[2]);
  if (ntok >= 2147483647.0) return fail(SWIN_ERR_UNSUPPORTED, "more than 2^31-1 tokens");
  if (ntok * double(d->channels) * 3.0 >= 9.2e18) return fail(SWIN_ERR_UNSUPPORTED, "tensor too large");
  return SWIN_OK;
}

// Split-K for a weight gradient (a contraction over n_tok tokens with an M x N output):
// 256 x 256 output tiles, one workgroup per CU at a time, and at most two full rounds of
// workgroups (no partial third round); chunks are whole 64-token steps.
void wgrad_split(int64_t n_tok, int64_t M, int64_t N, int* splits, int64_t* chunk) {
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  int64_t s = std::max<int64_t>(1, 512 / tiles);
  s = std::min<int64_t>(s, std::max<int64_t>(1, n_tok / 512));
  *splits = (int)s;
  const int64_t c = (n_tok + s - 1) / s;
  *chunk = (c + 63) / 64 * 64;
}

// Which kernels serve the descriptor: the one-tile bf16 path (head_dim 32, windows of up to
// 256 tokens, tables of up to 2048 bins), the tiled bf16 path (head_dim 32, 64 or 128, any
// window), or the fp32 forward path.
static swin_status check_kernel_support(const swin_attn_desc* d, int64_t max_tokens, bool* tiled) {
  const int hd = d->channels / d->heads;
  const int64_t nbins = int64_t(2 * d->window[0] - 1) * (2 * d->window[1] - 1) * (2 * d->window[2] - 1);
  *tiled = false;
  if (d->dtype == SWIN_BF16) {
    if (hd != 32 && hd != 64 && hd != 128)
      return fail(SWIN_ERR_UNSUPPORTED, "bf16 kernels need head_dim 32, 64 or 128");
    if (d->channels % 64 != 0) return fail(SWIN_ERR_UNSUPPORTED, "bf16 kernels need channels % 64 == 0");
    *tiled = hd != 32 || max_tokens > 16 * kMaxFwdTiles || nbins > kMaxBins;
    if (*tiled && nbins >= (int64_t(1) << 24))
      return fail(SWIN_ERR_UNSUPPORTED, "relative-position table of 2^24 bins or more per head");
  } else {
    if (max_tokens > 16 * kMaxFwdTiles)
      return fail(SWIN_ERR_UNSUPPORTED, "fp32 windows of more than 256 tokens are not supported");
    if (nbins > kMaxBins) return fail(SWIN_ERR_UNSUPPORTED, "relative-position table larger than 2048 bins per head");
    if (hd > 64) return fail(SWIN_ERR_UNSUPPORTED, "fp32 kernels need head_dim <= 64");
    if (2 * max_tokens * hd * 4 + max_tokens * 8 > 160 * 1024)
      return fail(SWIN_ERR_UNSUPPORTED, "fp32 window K/V tiles exceed the 160 KB of LDS");
  }
  return SWIN_OK;
}

// Host layout: everything the plan needs, without touching a device.
struct HostLayout {
  int64_t n_tok = 0, n_win = 0;
  std::vector<int32_t> perm;      // slot -> grid row
  std::vector<uint8_t> labels;    // slot -> label bits
  std::vector<int32_t> win_off;   // n_win + 1
  std::vector<int32_t> win_cls;   // window -> class
  std::vector<ClassInfo> classes;
  swin_attn_stats stats{};
};

static void build_layout(const swin_attn_desc* d, HostLayout& L) {
  const int64_t N[3] = {d->grid[0], d->grid[1], d->grid[2]};
  const int64_t w[3] = {d->window[0], d->window[1], d->window[2]};
  const int64_t s[3] = {d->shift[0], d->shift[1], d->shift[2]};
  int64_t nk[3];
  for (int a = 0; a < 3; ++a) nk[a] = (N[a] + w[a] - 1) / w[a];
  L.n_tok = d->batch * N[0] * N[1] * N[2];
  L.n_win = d->batch * nk[0] * nk[1] * nk[2];
  L.perm.resize(L.n_tok);
  L.labels.resize(L.n_tok);
  L.win_off.resize(L.n_win + 1);
  L.win_cls.resize(L.n_win);
  std::map<std::tuple<int, int, int, int, int, int>, int> cls_of;
  int64_t slot = 0, wi = 0, masked = 0, max_tok = 0, pairs = 0;
  for (int64_t b = 0; b < d->batch; ++b)
    for (int64_t kd = 0; kd < nk[0]; ++kd)
      for (int64_t kh = 0; kh < nk[1]; ++kh)
        for (int64_t kw = 0; kw < nk[2]; ++kw, ++wi) {
          const int64_t k[3] = {kd, kh, kw};
          int64_t start[3], ext[3], split[3];
          bool is_split = false;
          for (int a = 0; a < 3; ++a) {
            start[a] = k[a] * w[a];
            ext[a] = std::min(w[a], N[a] - start[a]);
            // rolled index r carries label 1 iff the axis is masked, s > 0 and r >= N - s
            split[a] = ext[a];
            if (!((d->periodic >> a) & 1u) && s[a] > 0) {
              const int64_t sp = N[a] - s[a] - start[a];
              if (sp > 0 && sp < ext[a]) {
                split[a] = sp;
                is_split = true;
              }
            }
          }
          const int64_t n = ext[0] * ext[1] * ext[2];
          L.win_off[wi] = (int32_t)slot;
          auto key = std::make_tuple((int)ext[0], (int)ext[1], (int)ext[2], (int)split[0], (int)split[1], (int)split[2]);
          auto it = cls_of.find(key);
          int c;
          if (it == cls_of.end()) {
            c = (int)L.classes.size();
            cls_of[key] = c;
            ClassInfo ci{};
            for (int a = 0; a < 3; ++a) {
              ci.ext[a] = (int32_t)ext[a];
              ci.split[a] = (int32_t)split[a];
            }
            ci.n = (int32_t)n;
            ci.nqt = (int32_t)((n + 15) / 16);
            L.classes.push_back(ci);
          } else {
            c = it->second;
          }
          L.win_cls[wi] = c;
          L.classes[c].count++;
          masked += is_split;
          max_tok = std::max(max_tok, n);
          int64_t lab_count[8] = {0};
          for (int64_t ld = 0; ld < ext[0]; ++ld)
            for (int64_t lh = 0; lh < ext[1]; ++lh)
              for (int64_t lw = 0; lw < ext[2]; ++lw, ++slot) {
                const int64_t r[3] = {start[0] + ld, start[1] + lh, start[2] + lw};
                int64_t o[3];
                uint8_t lab = 0;
                for (int a = 0; a < 3; ++a) {
                  o[a] = (r[a] + s[a]) % N[a];  // rolled index r holds original (r + s) mod N
                  if (!((d->periodic >> a) & 1u) && s[a] > 0 && r[a] >= N[a] - s[a]) lab |= uint8_t(1u << a);
                }
                L.perm[slot] = (int32_t)(((b * N[0] + o[0]) * N[1] + o[1]) * N[2] + o[2]);
                L.labels[slot] = lab;
                lab_count[lab]++;
              }
          for (int l = 0; l < 8; ++l) pairs += lab_count[l] * lab_count[l];
        }
  L.win_off[L.n_win] = (int32_t)slot;
  L.stats.n_tokens = L.n_tok;
  L.stats.n_windows = L.n_win;
  L.stats.n_masked = masked;
  L.stats.n_classes = (int64_t)L.classes.size();
  L.stats.max_tokens = max_tok;
  L.stats.allowed_pairs = pairs;
}

template <class T>
static hipError_t upload(T** dst, const std::vector<T>& src) {
  *dst = nullptr;
  if (src.empty()) return hipSuccess;
  hipError_t e = hipMalloc((void**)dst, src.size() * sizeof(T));
  if (e != hipSuccess) return e;
  return hipMemcpy(*dst, src.data(), src.size() * sizeof(T), hipMemcpyHostToDevice);
}

static void free_dev(swin_attn_plan* p) {
  if (p->device >= 0) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(p->device);
    hipFree(p->dev.perm);
    hipFree(p->dev.win_off);
    hipFree(p->dev.class_win);
    hipFree(p->dev.classes);
    hipFree(p->dev.fwd_work);
    hipFree(p->dev.bwd_work);
    hipFree(p->dev.tiled_work);
    hipFree(p->dev.tiled_kv_work);
    hipFree(p->dev.tiled_codes);
    hipFree(p->dev.flags);
    if (cur >= 0) (void)hipSetDevice(cur);
  }
  p->dev = DevTables{};
}

// Windows per workgroup: enough chunks to fill the chip several times over, few enough
// that per-class bias/mask setup is amortised.
// Work items grouped by tile count (one launch per count). Within a launch every class is cut
// into chunks of the same number of windows ch (each work item is one chunk for every head), and
// ch minimises rounds * (ch + ovh): rounds = ceil(items / slots) waves of workgroups over the
// launch's slots (CUs x workgroups per CU), ovh the fixed cost of a workgroup in windows (set-up,
// and in the backward the bias-gradient binning). A class of a few windows thus gets a few
// items instead of one per head per window; ties go to the smaller chunk (more items).
static void build_work(const std::vector<ClassInfo>& classes, int heads, int n_cu, int ovh, int cap,
                       const std::function<int(int)>& blocks_per_cu, std::vector<WorkItem>& out,
                       std::vector<WorkRange>& ranges) {
  out.clear();
  ranges.clear();
  for (int nqt = 16; nqt >= 1; --nqt) {
    std::vector<int> cls;
    for (int c = 0; c < (int)classes.size(); ++c)
      if (classes[c].nqt == nqt) cls.push_back(c);
    if (cls.empty()) continue;
    const int64_t slots = (int64_t)n_cu * blocks_per_cu(nqt);
    int best = 1;
    int64_t best_cost = -1;
    for (int ch = 1; ch <= cap; ++ch) {
      int64_t items = 0;
      for (int c : cls) items += (classes[c].count + ch - 1) / ch;
      const int64_t rounds = (items * heads + slots - 1) / slots;
      const int64_t cost = rounds * (ch + ovh);
      if (best_cost < 0 || cost < best_cost) {
        best_cost = cost;
        best = ch;
      }
    }
    const int begin = (int)out.size();
    for (int c : cls)
      for (int f = 0; f < classes[c].count; f += best) {
        WorkItem w{};
        w.cls = c;
        w.first = classes[c].first + f;
        w.count = std::min(best, classes[c].count - f);
        out.push_back(w);
      }
    ranges.push_back(WorkRange{nqt, begin, (int)out.size() - begin});
  }
}

// Argument checks of the module backward, shared by swin_attn_bwd and swin_attn_bwd_noalloc.
swin_status bwd_arg_checks(const swin_attn_plan* plan, const void* dy, const void* x, const void* w_qkv,
                           const void* w_proj, const float* bias_table, const void* saved, const void* dx,
                           const float* dw_qkv, const float* dw_proj, const float* dbias_table) {
  if (!plan) return fail(SWIN_ERR_ARG, "plan is NULL");
  if (plan->d.dtype != SWIN_BF16) return fail(SWIN_ERR_UNSUPPORTED, "backward is implemented for bf16 only");
  if (!dy || !x || !w_qkv || !w_proj || !bias_table || !saved || !dx || !dw_qkv || !dw_proj || !dbias_table)
    return fail(SWIN_ERR_ARG, "NULL input or output pointer");
  if (dx == dy || dx == x) return fail(SWIN_ERR_ARG, "dx must not alias dy or x");
  return SWIN_OK;
}

}  // namespace swin

using namespace swin;

extern "C" {

const char* swin_status_string(swin_status st) {
  switch (st) {
    case SWIN_OK: return "SWIN_OK";
    case SWIN_ERR_ARG: return "SWIN_ERR_ARG: invalid argument";
    case SWIN_ERR_UNSUPPORTED: return "SWIN_ERR_UNSUPPORTED: shape or dtype not supported";
    case SWIN_ERR_WORKSPACE: return "SWIN_ERR_WORKSPACE: workspace missing or too small";
    case SWIN_ERR_HIP: return "SWIN_ERR_HIP: HIP runtime error";
  }
  return "unknown swin_status";
}

const char* swin_attn_last_error(void) { return g_last_error.c_str(); }

swin_status swin_attn_trace_events(void* const* events, int capacity) {
  if (events && capacity < 0) return fail(SWIN_ERR_ARG, "negative trace capacity");
  g_trace.events = events;
  g_trace.capacity = events ? capacity : 0;
  g_trace.cursor = 0;
  return SWIN_OK;
}

int swin_attn_trace_cursor(void) { return g_trace.cursor; }

swin_status swin_attn_host_index_map(const swin_attn_desc* desc, int64_t* map, uint8_t* labels) {
  swin_status st = validate(desc);
  if (st != SWIN_OK) return st;
  HostLayout L;
  build_layout(desc, L);
  for (int64_t t = 0; t < L.n_tok; ++t) {
    if (map) map[t] = L.perm[t];
    if (labels) labels[t] = L.labels[t];
  }
  return SWIN_OK;
}

swin_status swin_attn_index_map(const swin_attn_plan* plan, int64_t* map, uint8_t* labels) {
  if (!plan) return fail(SWIN_ERR_ARG, "plan is NULL");
  for (int64_t t = 0; t < plan->n_tok; ++t) {
    if (map) map[t] = plan->perm[t];
    if (labels) labels[t] = plan->labels[t];
  }
  return SWIN_OK;
}

swin_status swin_attn_host_stats(const swin_attn_desc* desc, swin_attn_stats* out) {
  if (!out) return fail(SWIN_ERR_ARG, "stats output is NULL");
  swin_status st = validate(desc);
  if (st != SWIN_OK) return st;
  HostLayout L;
  build_layout(desc, L);
  *out = L.stats;
  return SWIN_OK;
}

swin_status swin_attn_plan_create(const swin_attn_desc* desc, swin_attn_plan** out) {
  if (!out) return fail(SWIN_ERR_ARG, "plan output is NULL");
  *out = nullptr;
  swin_status st = validate(desc);
  if (st != SWIN_OK) return st;
  HostLayout L;
  build_layout(desc, L);
  bool tiled = false;
  st = check_kernel_support(desc, L.stats.max_tokens, &tiled);
  if (st != SWIN_OK) return st;

  swin_attn_plan* p = new (std::nothrow) swin_attn_plan();
  if (!p) return fail(SWIN_ERR_ARG, "out of host memory");
  p->d = *desc;
  p->tiled = tiled;
  p->tiled_bwd = desc->dtype == SWIN_BF16 && (tiled || L.stats.max_tokens > 16 * kMaxBwdTiles);
  p->n_tok = L.n_tok;
  p->n_win = L.n_win;
  p->C = desc->channels;
  p->nh = desc->heads;
  p->hd = p->C / p->nh;
  p->nbins = (2 * desc->window[0] - 1) * (2 * desc->window[1] - 1) * (2 * desc->window[2] - 1);
  p->tau = desc->scale > 0.f ? desc->scale : 1.0f / std::sqrt((float)p->hd);
  p->stats = L.stats;
  p->perm = std::move(L.perm);
  p->labels = std::move(L.labels);
  p->win_off = std::move(L.win_off);
  p->classes = std::move(L.classes);
  // class-sorted window list (row-major order inside a class)
  {
    int f = 0;
    for (auto& c : p->classes) {
      c.first = f;
      f += c.count;
    }
    std::vector<int32_t> fill(p->classes.size(), 0);
    p->class_win.resize(p->n_win);
    for (int64_t w = 0; w < p->n_win; ++w) {
      const int c = L.win_cls[w];
      p->class_win[p->classes[c].first + fill[c]++] = (int32_t)w;
    }
  }
  // work items are sized for the current device's CU count (the plan is created on it)
  int n_cu = 0, cur_dev = 0;
  if (hipGetDevice(&cur_dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, cur_dev) != hipSuccess || n_cu < 1)
    n_cu = 256;
  build_work(p->classes, p->nh, n_cu, kFwdItemOverhead, kFwdMaxChunk, attn_fwd_blocks_per_cu, p->fwd_work,
             p->fwd_ranges);
  if (p->tiled || p->tiled_bwd) {
    // token-code tables of every class: key codes, then query codes, kCodeRound-padded
    const bool enc = p->nbins <= kTabLds;
    const int code0 = code0_of(desc->window);
    std::vector<int32_t> code_off(p->classes.size());
    for (size_t c = 0; c < p->classes.size(); ++c) {
      const ClassInfo& ci = p->classes[c];
      const int nr = (ci.n + kCodeRound - 1) / kCodeRound * kCodeRound;
      code_off[c] = (int32_t)p->tiled_codes.size();
      p->tiled_codes.resize(p->tiled_codes.size() + 2 * (size_t)nr);
      int32_t* kc = p->tiled_codes.data() + code_off[c];
      for (int j = 0; j < nr; ++j) {
        const int code = j < ci.n ? token_code(j, ci.ext, ci.split, desc->window) : 0;
        kc[j] = j < ci.n ? (enc ? enc_key(code) : code) : (enc ? kPadK : kPadCode);
        kc[nr + j] = j < ci.n ? (enc ? enc_query(code, code0) : code) : (enc ? kPadQ : kPadCode);
      }
    }
    // one item per 64-token block of every window, windows in row-major order
    for (int64_t w = 0; w < p->n_win; ++w) {
      const int n = p->win_off[w + 1] - p->win_off[w];
      const int c = L.win_cls[w];
      for (int b = 0; b * 64 < n; ++b) p->tiled_work.push_back(WorkItem{c, (int32_t)w, b, code_off[c]});
      for (int b = 0; b * 128 < n; ++b) p->tiled_kv_work.push_back(WorkItem{c, (int32_t)w, b, code_off[c]});
    }
  }
  // the backward ends every workgroup with a pass that bins its bias-gradient sums: a larger
  // fixed cost per workgroup than the forward's
  {
    const size_t dyn = 2 * (size_t)p->nbins * sizeof(float);
    build_work(p->classes, p->nh, n_cu, kBwdItemOverhead, kMaxChunk,
               [dyn](int nqt) { return nqt <= kMaxBwdTiles ? attn_bwd_blocks_per_cu(nqt, dyn) : 1; }, p->bwd_work,
               p->bwd_ranges);
  }

  // saved state and workspace layout
  const size_t es = desc->dtype == SWIN_BF16 ? 2 : 4;
  const size_t nt = (size_t)p->n_tok, C = (size_t)p->C;
  p->saved_qkv = align256(3 * nt * C * es);
  p->saved_o = align256(nt * C * es);
  p->saved_lse = align256(nt * (size_t)p->nh * 4);
  p->saved_total = p->saved_qkv + p->saved_o + p->saved_lse;
  if (desc->dtype == SWIN_BF16) {
    wgrad_split(p->n_tok, 3 * C, C, &p->wgrad_splits_qkv, &p->wgrad_chunk_qkv);
    wgrad_split(p->n_tok, C, C, &p->wgrad_splits_proj, &p->wgrad_chunk_proj);
    p->bwd_do = align256(nt * C * 2);
    p->bwd_dqkv = align256(nt * 3 * C * 2);
    p->bwd_wt = align256((C * C + 3 * C * C) * 2);
    const size_t part_qkv = (size_t)p->wgrad_splits_qkv * (3 * C * C + 3 * C);
    const size_t part_proj = (size_t)p->wgrad_splits_proj * (C * C + C);
    p->bwd_part = align256(std::max(part_qkv, part_proj) * 4);
    // dT: per-work-item partials (one-tile path) or one fixed-point accumulator (tiled path)
    p->bwd_dbias_part = p->tiled_bwd ? align256((size_t)p->nh * (size_t)p->nbins * 8 + 8)  // + saturation word
                                 : align256(p->bwd_work.size() * (size_t)p->nh * (size_t)p->nbins * 4);
    p->bwd_dd = align256(nt * (size_t)p->nh * 4);
    p->bwd_total = p->bwd_do + p->bwd_dqkv + p->bwd_wt + p->bwd_part + p->bwd_dbias_part + p->bwd_dd;
  }

  hipError_t e = hipGetDevice(&p->device);
  if (e == hipSuccess) e = upload(&p->dev.perm, p->perm);
  if (e == hipSuccess) e = upload(&p->dev.win_off, p->win_off);
  if (e == hipSuccess) e = upload(&p->dev.class_win, p->class_win);
  if (e == hipSuccess) e = upload(&p->dev.classes, p->classes);
  if (e == hipSuccess) e = upload(&p->dev.fwd_work, p->fwd_work);
  if (e == hipSuccess) e = upload(&p->dev.bwd_work, p->bwd_work);
  if (e == hipSuccess && !p->tiled_work.empty()) e = upload(&p->dev.tiled_work, p->tiled_work);
  if (e == hipSuccess && !p->tiled_kv_work.empty()) e = upload(&p->dev.tiled_kv_work, p->tiled_kv_work);
  if (e == hipSuccess && !p->tiled_codes.empty()) e = upload(&p->dev.tiled_codes, p->tiled_codes);
  if (e == hipSuccess) e = upload(&p->dev.flags, std::vector<unsigned int>{0u});
  if (e != hipSuccess) {
    set_error(std::string("plan upload failed: ") + hipGetErrorString(e));
    free_dev(p);
    delete p;
    return SWIN_ERR_HIP;
  }
  *out = p;
  return SWIN_OK;
}

void swin_attn_plan_destroy(swin_attn_plan* plan) {
  if (!plan) return;
  free_dev(plan);
  delete plan;
}

swin_status swin_attn_plan_stats(const swin_attn_plan* plan, swin_attn_stats* out) {
  if (!plan || !out) return fail(SWIN_ERR_ARG, "plan or output is NULL");
  *out = plan->stats;
  return SWIN_OK;
}

swin_status swin_attn_plan_flags(const swin_attn_plan* plan, uint32_t* flags, int clear) {
  if (!plan || !flags) return fail(SWIN_ERR_ARG, "plan or flags is NULL");
  if (!plan->dev.flags) return fail(SWIN_ERR_ARG, "plan has no device state (host-only plan)");
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e == hipSuccess) e = hipSetDevice(plan->device);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  unsigned int v = 0u;
  if (e == hipSuccess) e = hipMemcpy(&v, plan->dev.flags, sizeof(v), hipMemcpyDeviceToHost);
  const unsigned int zero = 0u;
  if (e == hipSuccess && clear) e = hipMemcpy(plan->dev.flags, &zero, sizeof(zero), hipMemcpyHostToDevice);
  if (cur >= 0) (void)hipSetDevice(cur);
  if (e != hipSuccess) {
    set_error(std::string("reading the plan flags: ") + hipGetErrorString(e));
    return SWIN_ERR_HIP;
  }
  *flags = v;
  return SWIN_OK;
}

swin_status swin_attn_sizes(const swin_attn_plan* plan, size_t* fwd_ws, size_t* bwd_ws, size_t* saved_bytes) {
  if (!plan) return fail(SWIN_ERR_ARG, "plan is NULL");
  if (fwd_ws) *fwd_ws = 0;
  if (bwd_ws) *bwd_ws = plan->bwd_total;
  if (saved_bytes) *saved_bytes = plan->saved_total;
  return SWIN_OK;
}

static swin_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SWIN_OK;
  set_error(std::string(what) + ": " + hipGetErrorString(e));
  return SWIN_ERR_HIP;
}

swin_status swin_window_gather(const swin_attn_plan* plan, const void* x, void* xw, void* stream) {
  if (!plan || !x || !xw) return fail(SWIN_ERR_ARG, "NULL plan or buffer");
  if (x == xw) return fail(SWIN_ERR_ARG, "gather cannot run in place");
  return hip_status(launch_gather(plan, x, xw, false, (hipStream_t)stream), "gather launch");
}

swin_status swin_window_scatter(const swin_attn_plan* plan, const void* yw, void* y, void* stream) {
  if (!plan || !yw || !y) return fail(SWIN_ERR_ARG, "NULL plan or buffer");
  if (yw == y) return fail(SWIN_ERR_ARG, "scatter cannot run in place");
  return hip_status(launch_gather(plan, yw, y, true, (hipStream_t)stream), "scatter launch");
}

swin_status swin_attn_fwd(const swin_attn_plan* plan, const void* x, const void* w_qkv, const void* b_qkv,
                          const void* w_proj, const void* b_proj, const float* bias_table, void* y, void* saved,
                          void* ws, size_t ws_bytes, void* stream) {
  if (!plan) return fail(SWIN_ERR_ARG, "plan is NULL");
  if (!x || !w_qkv || !w_proj || !bias_table || !y) return fail(SWIN_ERR_ARG, "NULL input or output pointer");
  if (x == y) return fail(SWIN_ERR_ARG, "y must not alias x");
  void* sv = saved;
  if (!sv) {
    if (!ws || ws_bytes < plan->saved_total)
      return fail(SWIN_ERR_WORKSPACE, "inference call needs a workspace of saved_bytes");
    sv = ws;
  }
  hipStream_t s = (hipStream_t)stream;
  if (plan->d.dtype == SWIN_F32)
    return hip_status(launch_fwd_f32(plan, x, w_qkv, b_qkv, w_proj, b_proj, bias_table, y, sv, s), "fp32 forward");
  char* base = (char*)sv;
  void* qkv = base;
  void* o = base + plan->saved_qkv;
  float* lse = (float*)(base + plan->saved_qkv + plan->saved_o);
  hipError_t e = trace_mark(s);
  if (e == hipSuccess) e = launch_qkv_fwd_bf16(plan, x, w_qkv, b_qkv, qkv, s);
  if (e == hipSuccess) e = trace_mark(s);
  if (e == hipSuccess) e = launch_attn_fwd_bf16(plan, qkv, bias_table, o, lse, s);
  if (e == hipSuccess) e = trace_mark(s);
  if (e == hipSuccess) e = launch_proj_fwd_bf16(plan, o, w_proj, b_proj, y, s);
  if (e == hipSuccess) e = trace_mark(s);
  return hip_status(e, "bf16 forward");
}

swin_status swin_attn_bwd(const swin_attn_plan* plan, const void* dy, const void* x, const void* w_qkv,
                          const void* w_proj, const float* bias_table, const void* saved, void* dx, float* dw_qkv,
                          float* db_qkv, float* dw_proj, float* db_proj, float* dbias_table, void* ws,
                          size_t ws_bytes, void* stream) {
  const swin_status st = bwd_arg_checks(plan, dy, x, w_qkv, w_proj, bias_table, saved, dx, dw_qkv, dw_proj,
                                        dbias_table);
  if (st != SWIN_OK) return st;
  if (!ws || ws_bytes < plan->bwd_total) return fail(SWIN_ERR_WORKSPACE, "backward workspace too small");
  return hip_status(launch_bwd_bf16(plan, dy, x, w_qkv, w_proj, bias_table, saved, dx, dw_qkv, db_qkv, dw_proj,
                                    db_proj, dbias_table, ws, (hipStream_t)stream),
                    "bf16 backward");
}

swin_status swin_attn_sizes_recompute(const swin_attn_plan* plan, size_t* fwd_ws, size_t* bwd_ws,
                                      size_t* saved_bytes) {
  if (!plan) return fail(SWIN_ERR_ARG, "plan is NULL");
  if (plan->d.dtype != SWIN_BF16) return fail(SWIN_ERR_UNSUPPORTED, "the recomputing calls are implemented for bf16 only");
  if (fwd_ws) *fwd_ws = plan->saved_qkv;
  if (bwd_ws) *bwd_ws = plan->saved_qkv + plan->bwd_total;
  if (saved_bytes) *saved_bytes = plan->saved_o + plan->saved_lse;
  return SWIN_OK;
}

swin_status swin_attn_fwd_recompute(const swin_attn_plan* plan, const void* x, const void* w_qkv, const void* b_qkv,
                                    const void* w_proj, const void* b_proj, const float* bias_table, void* y,
                                    void* saved, void* ws, size_t ws_bytes, void* stream) {
  if (!plan) return fail(SWIN_ERR_ARG, "plan is NULL");
  if (plan->d.dtype != SWIN_BF16) return fail(SWIN_ERR_UNSUPPORTED, "the recomputing calls are implemented for bf16 only");
  if (!x || !w_qkv || !w_proj || !bias_table || !y || !saved) return fail(SWIN_ERR_ARG, "NULL input or output pointer");
  if (x == y) return fail(SWIN_ERR_ARG, "y must not alias x");
  if (!ws || ws_bytes < plan->saved_qkv) return fail(SWIN_ERR_WORKSPACE, "forward workspace too small (q/k/v planes)");
  hipStream_t s = (hipStream_t)stream;
  void* qkv = ws;
  void* o = saved;
  float* lse = (float*)((char*)saved + plan->saved_o);
  hipError_t e = trace_mark(s);
  if (e == hipSuccess) e = launch_qkv_fwd_bf16(plan, x, w_qkv, b_qkv, qkv, s);
  if (e == hipSuccess) e = trace_mark(s);
  if (e == hipSuccess) e = launch_attn_fwd_bf16(plan, qkv, bias_table, o, lse, s);
  if (e == hipSuccess) e = trace_mark(s);
  if (e == hipSuccess) e = launch_proj_fwd_bf16(plan, o, w_proj, b_proj, y, s);
  if (e == hipSuccess) e = trace_mark(s);
  return hip_status(e, "bf16 forward (recomputing)");
}

swin_status swin_attn_bwd_recompute(const swin_attn_plan* plan, const void* dy, const void* x, const void* w_qkv,
                                    const void* b_qkv, const void* w_proj, const float* bias_table, const void* saved,
                                    void* dx, float* dw_qkv, float* db_qkv, float* dw_proj, float* db_proj,
                                    float* dbias_table, void* ws, size_t ws_bytes, void* stream) {
  const swin_status st = bwd_arg_checks(plan, dy, x, w_qkv, w_proj, bias_table, saved, dx, dw_qkv, dw_proj,
                                        dbias_table);
  if (st != SWIN_OK) return st;
  if (!ws || ws_bytes < plan->saved_qkv + plan->bwd_total)
    return fail(SWIN_ERR_WORKSPACE, "backward workspace too small (q/k/v planes + backward workspace)");
  hipStream_t s = (hipStream_t)stream;
  void* qkv = ws;
  const char* sv = (const char*)saved;
  // q/k/v again from x, by the forward's own GEMM (bitwise the planes the forward attended over)
  hipError_t e = launch_qkv_fwd_bf16(plan, x, w_qkv, b_qkv, qkv, s);
  if (e == hipSuccess)
    e = launch_bwd_bf16_parts(plan, dy, x, w_qkv, w_proj, bias_table, qkv, sv, (const float*)(sv + plan->saved_o), dx,
                              dw_qkv, db_qkv, dw_proj, db_proj, dbias_table, (char*)ws + plan->saved_qkv, s);
  return hip_status(e, "bf16 backward (recomputing q/k/v)");
}

swin_status swin_attn_bwd_noalloc(const swin_attn_plan* plan, const void* dy, const void* x, const void* w_qkv,
                                  const void* w_proj, const float* bias_table, const void* saved, void* dx,
                                  float* dw_qkv, float* db_qkv, float* dw_proj, float* db_proj, float* dbias_table,
                                  void* stream) {
  const swin_status st = bwd_arg_checks(plan, dy, x, w_qkv, w_proj, bias_table, saved, dx, dw_qkv, dw_proj,
                                        dbias_table);
  if (st != SWIN_OK) return st;
  if (plan->bwd_total > SWIN_NOALLOC_SCRATCH_BYTES)
    return fail(SWIN_ERR_WORKSPACE, "backward workspace of " + std::to_string(plan->bwd_total) +
                                        " bytes exceeds the " + std::to_string(SWIN_NOALLOC_SCRATCH_BYTES) +
                                        "-byte scratch of swin_attn_bwd_noalloc; use swin_attn_bwd");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev != plan->device) return fail(SWIN_ERR_ARG, "the current device is not the plan's device");
  void* ws = nullptr;
  e = noalloc_scratch(dev, &ws);
  if (e == hipSuccess)
    e = launch_bwd_bf16(plan, dy, x, w_qkv, w_proj, bias_table, saved, dx, dw_qkv, db_qkv, dw_proj, db_proj,
                        dbias_table, ws, (hipStream_t)stream);
  return hip_status(e, "bf16 backward (no allocation)");
}

}  // extern "C"
