"""Throughput of shifted-window attention forward + backward on one MI355X.

One step = the whole hot path on the 540x1080-token, C=512, 16-head, 12x12-window
workload (a 2160x4320 field after 4x4 patch embedding): W-MSA forward, SW-MSA
(shift 6,6) forward, SW-MSA backward, W-MSA backward, each module being gather +
QKV GEMM + window attention + proj GEMM + scatter and their backward. Inputs are
seeded synthetic data resident in HBM before the timed region. After the timed steps the
window gather and scatter are also timed stand-alone against a device-to-device copy, and the
chain is timed on one GPU's share of an 8-way latitude split (72x1080 tokens), with the saved
state sent to host memory and back, and on the recomputing calls (o + LSE saved, q/k/v rebuilt
in each backward).

Then the other workloads of the measurement plan, each on its own (180x360 batch 2, the ragged
181x361 grid and the 8x180x360 level grid forward + backward; the 32x64 fp32 grid forward):
median / min / max over 50 calls after 10 warm-ups, then the same over 50 replays of the calls
captured once in a HIP graph (graph_replay: no per-call host work), with the fp64 oracle timed
on the same inputs (and the brute-force per-token loop on the fp32 grid).

Prints one JSON line on stdout:
  value = token-blocks per second (tokens x modules per step / step time),
  tflops / mfma_peak_frac = algorithmic FLOPs per second and their fraction of the
  dense bf16 MFMA peak, step_ms = median / min / max of the timed steps,
  hbm_bytes_per_step = the algorithmic bytes of all stages of a step,
  roofline = the dominant kernel against its bound (stage durations from HIP events the
  library records between stages, in a second pass of the same number of steps after the
  timed one, which records events only at step boundaries),
  configs = the other workloads, cpu_baseline = the fp64 oracle on a bounded sample of the
  same workload (CPU model and BLAS threads recorded).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--cpu-seconds S]
"""
import argparse
import ctypes
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12   # 256 CUs x 4096 dense bf16 FLOP/clk x 2.4 GHz = 2516.6
PEAK_HBM_GBS = 8000.0
METRIC = "window-attn fwd+bwd tokens/s and TFLOPS (% of MI355X bf16 MFMA peak)"

FWD_STAGES = ["qkv_gemm", "attn_fwd", "proj_gemm"]
BWD_STAGES = ["w_transpose", "dproj_gemm", "wgrad_proj", "attn_bwd", "dbias_reduce", "dgrad_qkv", "wgrad_qkv"]
# stage -> (kernel name as rocprofv3 reports it, source file) for the single-kernel stages
STAGE_KERNEL = {
    "qkv_gemm": ("k_gemm_nt_wide<false>", "gemm.hip"), "proj_gemm": ("k_gemm_nt", "gemm.hip"),
    "dproj_gemm": ("k_gemm_nt_wide<true>", "gemm.hip"), "dgrad_qkv": ("k_gemm_nt", "gemm.hip"),
    "attn_fwd": ("k_attn_fwd", "attn_fwd.hip"), "attn_bwd": ("k_attn_bwd", "attn_bwd.hip"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """The few HIP runtime calls the bench needs for events."""

    def __init__(self):
        self.l = ctypes.CDLL("libamdhip64.so")
        self.l.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.l.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.l.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.l.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            assert self.l.hipEventCreate(ctypes.byref(h)) == 0
            arr[i] = h
        return arr

    def elapsed_ms(self, a, b):
        f = ctypes.c_float()
        assert self.l.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return float(f.value)

    def destroy(self, arr):
        for h in arr:
            self.l.hipEventDestroy(h)


def stage_flops_bytes(cfg, pairs):
    """Algorithmic FLOPs and HBM bytes per launch of each stage for one module."""
    N, C, nh, hd = cfg.n_tokens, cfg.channels, cfg.heads, cfg.head_dim
    core = 4 * hd * pairs * nh
    tok_head = N * nh
    f = {"qkv_gemm": 2 * N * C * 3 * C, "attn_fwd": core, "proj_gemm": 2 * N * C * C,
         "w_transpose": 0, "dproj_gemm": 2 * N * C * C, "wgrad_proj": 2 * N * C * C, "attn_bwd": 2 * core,
         "dbias_reduce": 0, "dgrad_qkv": 2 * N * 3 * C * C, "wgrad_qkv": 2 * N * 3 * C * C}
    # bytes the stage must move as designed: operands in, results out (bf16 = 2 B)
    b = {"qkv_gemm": 2 * N * C + 2 * N * 3 * C,                     # x in, q/k/v out
         "attn_fwd": tok_head * (3 * 64 + 64 + 4),                  # q, k, v in; o, lse out
         "proj_gemm": 2 * N * C * 2,                                # o in, y out
         "dproj_gemm": 2 * N * C * 3 + tok_head * 4,                # dy, o in; dO, D = rowsum(dO o) out
         "wgrad_proj": 2 * N * C * 2,                               # dy, o in
         "attn_bwd": tok_head * (4 * 64 + 2 * 4 + 3 * 64),          # q k v dO lse D in; dq dk dv out
         "dgrad_qkv": 2 * N * 3 * C + 2 * N * C,                    # dqkv in, dx out
         "wgrad_qkv": 2 * N * 3 * C + 2 * N * C,                    # dqkv, x in
         "w_transpose": 2 * 2 * 4 * C * C, "dbias_reduce": 0}
    return f, b


def source_sha(fname):
    """Hash of a kernel source file's code: comments and blank lines are left out, so that a
    change of comments alone does not mark counters taken on the file as stale. (bench.py and
    profile_summary.py compute it the same way.)"""
    with open(os.path.join(ROOT, "shifted_window_attention_amd", "csrc", fname)) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_for(stage, per_launch_ref):
    """HBM bytes per launch from committed rocprofv3 PMC counters, if they were taken on the
    current kernel source (else None)."""
    kern = STAGE_KERNEL.get(stage)
    if not kern:
        return None
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except ValueError:
        return None
    rec = data.get(stage)
    if not rec or rec.get("source_sha") != source_sha(kern[1]):
        return None
    return rec.get("bytes_per_launch")


def cpu_info():
    """CPU model name, visible cores and the BLAS library's thread count."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    threads = os.cpu_count() or 1
    try:
        import threadpoolctl
        info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if info:
            threads = max(int(i.get("num_threads", 1)) for i in info)
    except Exception:
        pass
    return {"model": model, "cores_visible": os.cpu_count() or 0, "blas_threads": int(threads)}


def cpu_baseline_sampled(cfg, params_f64, x_rows, dy_rows, lays, seconds, rng_seed=11):
    """The fp64 oracle, as it is, on random whole windows of every module of `cfg`, forward and
    forward + backward, until ~`seconds` of CPU work each. x_rows / dy_rows(mi) give the
    window-major float64 rows of module mi's input / upstream gradient for a list of window ids."""
    import numpy as np
    from oracle import swin_oracle as O
    rng = np.random.default_rng(rng_seed)
    res = {}
    for mode in ("fwd", "fwd_bwd"):
        tokens = windows = 0
        elapsed = 0.0
        while elapsed < seconds:
            for mi, lay in enumerate(lays):
                ids = sorted(rng.choice(len(lay.windows), min(4, len(lay.windows)), replace=False).tolist())
                xw = x_rows(mi, ids)
                dyw = dy_rows(mi, ids) if mode == "fwd_bwd" else None
                t0 = time.perf_counter()
                O.windows_fwd(xw, params_f64[mi], lay, cfg.heads, window_ids=ids)
                if mode == "fwd_bwd":
                    O.windows_bwd(dyw, xw, params_f64[mi], lay, cfg.heads, window_ids=ids)
                elapsed += time.perf_counter() - t0
                tokens += sum(lay.windows[i].n for i in ids)
                windows += len(ids)
        res[mode] = {"tokens_per_s": round(tokens / elapsed, 1), "windows": windows, "seconds": round(elapsed, 2)}
    return res


def cpu_baseline(cfg, inp, seconds):
    """The fp64 oracle, as it is, on whole windows of both modules of the headline workload."""
    from oracle import swin_oracle as O
    lays = [O.window_layout(cfg.batch, cfg.grid, cfg.window, s, cfg.periodic) for s in cfg.shifts]
    ps = [O.Params(m.w_qkv, m.b_qkv, m.w_proj, m.b_proj, m.table) for m in inp.modules]
    xws = [O.gather(inp.x, lay) for lay in lays]
    dyws = [O.gather(inp.dy, lay) for lay in lays]
    r = cpu_baseline_sampled(cfg, ps, lambda mi, ids: xws[mi], lambda mi, ids: dyws[mi], lays, seconds / 2)
    ci = cpu_info()
    fb = r["fwd_bwd"]
    return {"value": fb["tokens_per_s"], "unit": "tokens/s", "cores": ci["blas_threads"], "kind": "oracle",
            "sample": "%d random whole windows (fwd+bwd, float64 oracle) split over the W-MSA and SW-MSA modules "
                      "of the 540x1080 C=512 workload, %.1f s of CPU work (the full-grid gather is outside the "
                      "timed part); forward alone: %.1f tokens/s over %d windows; CPU %s, %d cores visible, "
                      "BLAS threads %d" % (fb["windows"], fb["seconds"], r["fwd"]["tokens_per_s"],
                                           r["fwd"]["windows"], ci["model"], ci["cores_visible"],
                                           ci["blas_threads"]),
            "seconds": fb["seconds"], "fwd_tokens_per_s": r["fwd"]["tokens_per_s"], "cpu": ci}


def _device_inputs(cfg):
    """Inputs of the same shapes and scales as the seeded recipe, drawn on the GPU."""
    import types
    import numpy as np
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    C = cfg.channels
    D, H, W = cfg.grid
    shape = (cfg.batch, D, H, W, C)

    def bits(t):
        return t.to(torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    mods = []
    for _ in range(cfg.modules):
        wq = torch.randn(3 * C, C, device="cuda", generator=g) * (2.0 / (4 * C)) ** 0.5
        wp = torch.randn(C, C, device="cuda", generator=g) * (1.0 / C) ** 0.5
        t = (torch.randn(cfg.bias_table_shape(), device="cuda", generator=g) * 0.02).cpu().numpy()
        mods.append(types.SimpleNamespace(w_qkv_dev=bits(wq), b_qkv_dev=np.zeros(3 * C, np.uint16),
                                          w_proj_dev=bits(wp), b_proj_dev=np.zeros(C, np.uint16), table_dev=t))
    x = torch.randn(shape, device="cuda", generator=g).to(torch.bfloat16)
    dy = torch.randn(shape, device="cuda", generator=g).to(torch.bfloat16)
    return types.SimpleNamespace(modules=mods, x_t=x, dy_t=dy)


PEAK_F32_TFLOPS = 157.3   # MI355X fp32 vector peak (the fp32 path runs on FMA, not MFMA)


def time_config(hip, N, stream, name, calls=50, warmup=10, cpu_seconds=2.0, with_cpu=True):
    """One workload of the measurement plan on its own: every module forward (and backward in
    reverse, for the bf16 workloads), `warmup` untimed calls, then `calls` calls each bracketed
    by HIP events on the library's stream; median / min / max per call. bf16 inputs are drawn on
    the device (seeded, same shapes and scales as the host recipe); the fp32 tiny workload uses
    the host recipe. The fp64 oracle is timed on random whole windows of the same inputs (and the
    brute-force per-token loop on the tiny workload)."""
    import numpy as np
    import torch
    from shifted_window_attention_amd.device import ModuleOnDevice, from_dev, to_dev
    from workloads import bf16_bits_to_f64, get_config, make_inputs
    cfg = get_config(name)
    f32 = cfg.dtype == "f32"
    if f32:
        inp = make_inputs(cfg, bias_scale=0.0)
        x = to_dev(inp.x_dev, "f32")
        dy = None
        params = inp.modules
    else:
        inp = _device_inputs(cfg)
        x, dy = inp.x_t, inp.dy_t
        params = inp.modules
    mods = [ModuleOnDevice(cfg, i, p) for i, p in enumerate(params)]
    C = cfg.channels
    ys = [torch.empty_like(x) for _ in mods]
    dxs = [torch.empty_like(x) for _ in mods] if cfg.backward else []
    grads = [{"w_qkv": torch.empty(3 * C, C, dtype=torch.float32, device="cuda"),
              "b_qkv": torch.empty(3 * C, dtype=torch.float32, device="cuda"),
              "w_proj": torch.empty(C, C, dtype=torch.float32, device="cuda"),
              "b_proj": torch.empty(C, dtype=torch.float32, device="cuda"),
              "table": torch.empty_like(m.table)} for m in mods] if cfg.backward else []

    def call(s=stream):
        xin = x
        for m, y in zip(mods, ys):
            N.swin_attn_fwd(m.plan.handle, xin, m.w_qkv, m.b_qkv, m.w_proj, m.b_proj, m.table, y, m.saved,
                            stream=s)
            xin = y
        if cfg.backward:
            d = dy
            for i in reversed(range(len(mods))):
                m, g = mods[i], grads[i]
                xin = x if i == 0 else ys[i - 1]
                N.swin_attn_bwd(m.plan.handle, d, xin, m.w_qkv, m.w_proj, m.table, m.saved, dxs[i], g["w_qkv"],
                                g["b_qkv"], g["w_proj"], g["b_proj"], g["table"], m.ws, stream=s)
                d = dxs[i]

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = hip.events(2 * calls)
    for i in range(calls):
        assert hip.l.hipEventRecord(ev[2 * i], stream.cuda_stream) == 0
        call()
        assert hip.l.hipEventRecord(ev[2 * i + 1], stream.cuda_stream) == 0
    torch.cuda.synchronize()
    ms = np.array([hip.elapsed_ms(ev[2 * i], ev[2 * i + 1]) for i in range(calls)])
    # the same calls captured once in a HIP graph (torch's graph API over the library's stream) and
    # replayed: the device time without per-call host work in the way
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        call(side)
    stream.wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call(side)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            graph.replay()
        for i in range(calls):
            assert hip.l.hipEventRecord(ev[2 * i], stream.cuda_stream) == 0
            graph.replay()
            assert hip.l.hipEventRecord(ev[2 * i + 1], stream.cuda_stream) == 0
    torch.cuda.synchronize()
    gms = np.array([hip.elapsed_ms(ev[2 * i], ev[2 * i + 1]) for i in range(calls)])
    del graph
    hip.destroy(ev)
    flops = 0
    for m in mods:
        f, _ = stage_flops_bytes(cfg, m.plan.stats["allowed_pairs"])
        flops += sum(f[s] for s in FWD_STAGES) + (sum(f[s] for s in BWD_STAGES) if cfg.backward else 0)
    med = float(np.median(ms))
    tfl = flops / (med * 1e-3) / 1e12
    res = {"config": cfg.description, "pass": "fwd+bwd" if cfg.backward else "fwd", "dtype": cfg.dtype,
           "tokens": cfg.n_tokens, "modules": cfg.modules, "calls": calls, "warmup": warmup,
           "median_ms": round(med, 4), "min_ms": round(float(ms.min()), 4), "max_ms": round(float(ms.max()), 4),
           "tokens_per_s": round(cfg.n_tokens * cfg.modules / (med * 1e-3), 1),
           "algorithmic_gflop": round(flops / 1e9, 3), "tflops": round(tfl, 2),
           "inputs": "host recipe (seed 0)" if f32 else "device-drawn (seeded torch generator, recipe's scales)"}
    if f32:
        res["fp32_peak_frac"] = round(tfl / PEAK_F32_TFLOPS, 5)
    else:
        res["mfma_peak_frac"] = round(tfl / PEAK_BF16_TFLOPS, 4)
    gmed = float(np.median(gms))
    res["graph_replay"] = {"median_ms": round(gmed, 4), "min_ms": round(float(gms.min()), 4),
                           "max_ms": round(float(gms.max()), 4),
                           "tokens_per_s": round(cfg.n_tokens * cfg.modules / (gmed * 1e-3), 1),
                           "tflops": round(flops / (gmed * 1e-3) / 1e12, 2)}
    if with_cpu:
        from oracle import swin_oracle as O
        lays = [O.window_layout(cfg.batch, cfg.grid, cfg.window, s, cfg.periodic) for s in cfg.shifts]
        if f32:
            ps = [O.Params(pm.w_qkv, pm.b_qkv, pm.w_proj, pm.b_proj, pm.table) for pm in params]
            xh = inp.x
            dyh = None
        else:
            def f64(bits):
                return bf16_bits_to_f64(bits)
            ps = [O.Params(f64(pm.w_qkv_dev), f64(pm.b_qkv_dev), f64(pm.w_proj_dev), f64(pm.b_proj_dev),
                           np.asarray(pm.table_dev, dtype=np.float64)) for pm in params]
            xh = from_dev(x)
            dyh = from_dev(dy)
        if cfg.modules == 1:
            xw = O.gather(xh, lays[0])
            dyw = O.gather(dyh, lays[0]) if dyh is not None else None
            if cfg.backward:
                r = cpu_baseline_sampled(cfg, ps, lambda mi, ids: xw, lambda mi, ids: dyw, lays, cpu_seconds)
            else:
                t0 = time.perf_counter()
                O.module_fwd(xh, ps[0], lays[0], cfg.heads)
                el = time.perf_counter() - t0
                r = {"fwd": {"tokens_per_s": round(cfg.n_tokens / el, 1), "windows": len(lays[0].windows),
                             "seconds": round(el, 3)}}
            if name == "tiny":
                t0 = time.perf_counter()
                O.brute_force_fwd(xh, ps[0], cfg.grid, cfg.window, cfg.shifts[0], cfg.periodic, cfg.heads)
                el = time.perf_counter() - t0
                r["brute_force_fwd"] = {"tokens_per_s": round(cfg.n_tokens / el, 1), "seconds": round(el, 2)}
            res["cpu_oracle"] = r
    for m in mods:
        m.plan.close()
    return res


def time_window_moves(hip, N, plan, x, stream, cfg, reps=20):
    """Stand-alone window gather (shift + partition) and scatter (reverse + un-shift) of the
    SW-MSA module, outside the timed step, against a device-to-device copy of the same bytes.
    The gather is also the known-size copy that calibrates the HBM byte counters."""
    import torch
    xw = torch.empty_like(x)
    y = torch.empty_like(x)
    ev = hip.events(2 * reps + 2)
    N.swin_window_gather(plan, x, xw, stream=stream)
    torch.cuda.synchronize()
    res = {}
    for name, fn in (("gather", lambda: N.swin_window_gather(plan, x, xw, stream=stream)),
                     ("scatter", lambda: N.swin_window_scatter(plan, xw, y, stream=stream)),
                     ("device_copy", lambda: y.copy_(xw))):
        for i in range(reps):
            assert hip.l.hipEventRecord(ev[2 * i], stream.cuda_stream) == 0
            fn()
            assert hip.l.hipEventRecord(ev[2 * i + 1], stream.cuda_stream) == 0
        torch.cuda.synchronize()
        ms = sorted(hip.elapsed_ms(ev[2 * i], ev[2 * i + 1]) for i in range(reps))[reps // 2]
        moved = 2 * x.numel() * x.element_size()   # read + write of the activation
        res[name] = {"median_ms": round(ms, 4), "gbs": round(moved / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(moved / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    hip.destroy(ev)
    for name in ("gather", "scatter"):
        res[name]["frac_of_device_copy"] = round(res[name]["gbs"] / res["device_copy"]["gbs"], 3)
    res["bytes_moved"] = 2 * x.numel() * x.element_size()
    return res


def time_shard_share(hip, N, stream, base_cfg, steps, warmup):
    """The same W-MSA -> SW-MSA chain on one GPU's share of an 8-way latitude split of the grid:
    72 of the 540 latitude rows (6 window rows, 540 windows per module). A sharded run would fill
    6 halo rows from the neighbour for the shifted module; here the stripe edges are masked like
    the grid's own latitude edges, so the per-GPU compute shape is the same."""
    import numpy as np
    import torch
    from shifted_window_attention_amd.device import ModuleOnDevice
    from workloads.configs import small_variant
    cfg = small_variant(base_cfg, grid=(1, 72, base_cfg.grid[2]))
    inp = _device_inputs(cfg)
    x, dy = inp.x_t, inp.dy_t
    mods = [ModuleOnDevice(cfg, i, p) for i, p in enumerate(inp.modules)]
    C = cfg.channels
    y1, y2, dx2, dx1 = (torch.empty_like(x) for _ in range(4))
    grads = [{"w_qkv": torch.empty(3 * C, C, dtype=torch.float32, device="cuda"),
              "b_qkv": torch.empty(3 * C, dtype=torch.float32, device="cuda"),
              "w_proj": torch.empty(C, C, dtype=torch.float32, device="cuda"),
              "b_proj": torch.empty(C, dtype=torch.float32, device="cuda"),
              "table": torch.empty_like(m.table)} for m in mods]

    def step():
        m1, m2 = mods
        N.swin_attn_fwd(m1.plan.handle, x, m1.w_qkv, m1.b_qkv, m1.w_proj, m1.b_proj, m1.table, y1, m1.saved,
                        stream=stream)
        N.swin_attn_fwd(m2.plan.handle, y1, m2.w_qkv, m2.b_qkv, m2.w_proj, m2.b_proj, m2.table, y2, m2.saved,
                        stream=stream)
        g = grads[1]
        N.swin_attn_bwd(m2.plan.handle, dy, y1, m2.w_qkv, m2.w_proj, m2.table, m2.saved, dx2, g["w_qkv"],
                        g["b_qkv"], g["w_proj"], g["b_proj"], g["table"], m2.ws, stream=stream)
        g = grads[0]
        N.swin_attn_bwd(m1.plan.handle, dx2, x, m1.w_qkv, m1.w_proj, m1.table, m1.saved, dx1, g["w_qkv"],
                        g["b_qkv"], g["w_proj"], g["b_proj"], g["table"], m1.ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = hip.events(2)
    assert hip.l.hipEventRecord(t0, stream.cuda_stream) == 0
    for _ in range(steps):
        step()
    assert hip.l.hipEventRecord(t1, stream.cuda_stream) == 0
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(t0, t1) / steps
    hip.destroy([t0, t1])
    flops = 0
    for m in mods:
        f, _ = stage_flops_bytes(cfg, m.plan.stats["allowed_pairs"])
        flops += sum(f.values())
    res = {"grid": list(cfg.grid[1:]), "windows_per_module": int(mods[0].plan.stats["n_windows"]),
           "tokens": cfg.n_tokens, "steps": steps, "ms_per_step": round(ms, 4),
           "tokens_per_s": round(cfg.n_tokens * cfg.modules / (ms * 1e-3), 1),
           "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
           "mfma_peak_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    for m in mods:
        m.plan.close()
    return res


def time_offload(hip, N, stream, mods, x, dy, outs, grads, steps):
    """The W-MSA module's saved state (q/k/v, o, LSE) sent to pinned host memory and back by the
    offload engine: each direction alone (GB/s), and the chain step with the store issued right
    after the W-MSA forward (overlapping the SW-MSA forward and backward) and the load issued
    before the W-MSA backward."""
    import torch
    m1, m2 = mods
    y1, y2, dx2, dx1 = outs
    nbytes = m1.plan.saved_bytes
    host = N.PinnedBuffer(nbytes)
    eng = N.swin_offload_create(0)
    ev = hip.events(2)
    res = {"saved_bytes": nbytes}
    for name, issue in (("store", lambda: N.swin_offload_store(eng, m1.saved, host, nbytes, after=stream)),
                        ("load", lambda: N.swin_offload_load(eng, host, m1.saved, nbytes, after=stream))):
        torch.cuda.synchronize()
        assert hip.l.hipEventRecord(ev[0], stream.cuda_stream) == 0
        t = issue()
        N.swin_offload_wait(eng, t, stream)
        assert hip.l.hipEventRecord(ev[1], stream.cuda_stream) == 0
        torch.cuda.synchronize()
        ms = hip.elapsed_ms(ev[0], ev[1])
        res[name + "_ms"] = round(ms, 3)
        res[name + "_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 2)

    def step():
        N.swin_attn_fwd(m1.plan.handle, x, m1.w_qkv, m1.b_qkv, m1.w_proj, m1.b_proj, m1.table, y1, m1.saved,
                        stream=stream)
        ts = N.swin_offload_store(eng, m1.saved, host, nbytes, after=stream)
        N.swin_attn_fwd(m2.plan.handle, y1, m2.w_qkv, m2.b_qkv, m2.w_proj, m2.b_proj, m2.table, y2, m2.saved,
                        stream=stream)
        g = grads[1]
        N.swin_attn_bwd(m2.plan.handle, dy, y1, m2.w_qkv, m2.w_proj, m2.table, m2.saved, dx2, g["w_qkv"],
                        g["b_qkv"], g["w_proj"], g["b_proj"], g["table"], m2.ws, stream=stream)
        N.swin_offload_wait(eng, ts, stream)
        tl = N.swin_offload_load(eng, host, m1.saved, nbytes, after=stream)
        N.swin_offload_wait(eng, tl, stream)
        g = grads[0]
        N.swin_attn_bwd(m1.plan.handle, dx2, x, m1.w_qkv, m1.w_proj, m1.table, m1.saved, dx1, g["w_qkv"],
                        g["b_qkv"], g["w_proj"], g["b_proj"], g["table"], m1.ws, stream=stream)

    step()
    torch.cuda.synchronize()
    assert hip.l.hipEventRecord(ev[0], stream.cuda_stream) == 0
    for _ in range(steps):
        step()
    assert hip.l.hipEventRecord(ev[1], stream.cuda_stream) == 0
    torch.cuda.synchronize()
    res["steps"] = steps
    res["chain_ms_per_step_with_offload"] = round(hip.elapsed_ms(ev[0], ev[1]) / steps, 3)
    hip.destroy(ev)
    N.swin_offload_destroy(eng)
    host.free()
    return res


def time_recompute(hip, N, stream, mods, x, dy, outs, grads, steps):
    """The chain step on the recomputing calls (saved state o + LSE; each backward rebuilds q/k/v
    from its input with the QKV GEMM): ms per step and the device memory that stays saved from the
    forwards to the backwards, against the saved-q/k/v calls."""
    import torch
    m1, m2 = mods
    y1, y2, dx2, dx1 = outs
    sizes = [N.swin_attn_sizes_recompute(m.plan.handle) for m in mods]
    saved = [torch.empty(sz[2], dtype=torch.uint8, device="cuda") for sz in sizes]
    ws = torch.empty(max(max(sz[0], sz[1]) for sz in sizes), dtype=torch.uint8, device="cuda")

    def step():
        N.swin_attn_fwd_recompute(m1.plan.handle, x, m1.w_qkv, m1.b_qkv, m1.w_proj, m1.b_proj, m1.table, y1,
                                  saved[0], ws, stream=stream)
        N.swin_attn_fwd_recompute(m2.plan.handle, y1, m2.w_qkv, m2.b_qkv, m2.w_proj, m2.b_proj, m2.table, y2,
                                  saved[1], ws, stream=stream)
        for m, d, xin, dxo, g, sv in ((m2, dy, y1, dx2, grads[1], saved[1]), (m1, dx2, x, dx1, grads[0], saved[0])):
            N.swin_attn_bwd_recompute(m.plan.handle, d, xin, m.w_qkv, m.b_qkv, m.w_proj, m.table, sv, dxo,
                                      g["w_qkv"], g["b_qkv"], g["w_proj"], g["b_proj"], g["table"], ws,
                                      stream=stream)

    ev = hip.events(2)
    step()
    torch.cuda.synchronize()
    assert hip.l.hipEventRecord(ev[0], stream.cuda_stream) == 0
    for _ in range(steps):
        step()
    assert hip.l.hipEventRecord(ev[1], stream.cuda_stream) == 0
    torch.cuda.synchronize()
    res = {"steps": steps, "chain_ms_per_step": round(hip.elapsed_ms(ev[0], ev[1]) / steps, 3),
           "saved_bytes_per_module": sizes[0][2], "saved_bytes_per_module_with_qkv": m1.plan.saved_bytes,
           "transient_workspace_bytes": ws.numel()}
    hip.destroy(ev)
    del saved, ws
    return res


def time_routes(hip, N, stream, cfg, ranks=8, reps=10):
    """TERRA's DMP route (8 latitude stripes -> 8 Eq. 4 window ranks) and shift route (unshifted
    -> shifted window ranks) on the full grid, all ranks on this GPU: per-rank pack, the
    loopback exchange of every segment, per-rank restore. Algorithmic bytes: each phase reads
    and writes every token row once (2 N C 2 B); the tokens that change rank are what a
    multi-GPU run would send over xGMI."""
    import numpy as np
    import torch
    C = cfg.channels
    gdesc = N.make_desc(cfg.batch, cfg.grid, C, 1, cfg.window, (0, 0, 0), cfg.periodic, N.SWIN_BF16)
    shift = cfg.shifts[-1]
    routes = {"dmp_route": (N.make_rank_layout(0, ranks), N.make_rank_layout(1, ranks)),
              "shift_route": (N.make_rank_layout(1, ranks), N.make_rank_layout(1, ranks, shift))}
    res = {"ranks": ranks}
    row = C * 2
    for name, (src, dst) in routes.items():
        plan = N.RoutePlan(gdesc, src, dst)
        locs = [torch.randn(int(n), C, device="cuda").to(torch.bfloat16) for n in plan.src_sizes]
        sends = [torch.empty_like(t) for t in locs]
        recvs = [torch.empty(int(n), C, dtype=torch.bfloat16, device="cuda") for n in plan.dst_sizes]
        outs = [torch.empty_like(t) for t in recvs]
        phases = {"pack": lambda: [N.swin_route_pack(plan, p, locs[p], sends[p], stream) for p in range(plan.P)],
                  "exchange": lambda: N.swin_route_loopback(plan, sends, recvs, stream),
                  "unpack": lambda: [N.swin_route_unpack(plan, r, recvs[r], outs[r], stream) for r in range(plan.R)]}
        rec = {}
        n_tok = int(plan.src_sizes.sum())
        for ph, fn in phases.items():
            fn()
            torch.cuda.synchronize()
            ev = hip.events(2)
            assert hip.l.hipEventRecord(ev[0], stream.cuda_stream) == 0
            for _ in range(reps):
                fn()
            assert hip.l.hipEventRecord(ev[1], stream.cuda_stream) == 0
            torch.cuda.synchronize()
            ms = hip.elapsed_ms(ev[0], ev[1]) / reps
            hip.destroy(ev)
            gbs = 2 * n_tok * row / (ms * 1e-3) / 1e9
            rec[ph] = {"ms": round(ms, 4), "gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
        moved = int(plan.counts.sum() - np.trace(plan.counts))
        rec["tokens_between_ranks"] = moved
        rec["mb_between_ranks"] = round(moved * row / 1e6, 1)
        rec["max_mb_per_rank_pair"] = round(
            float(max(plan.counts[p, r] for p in range(plan.P) for r in range(plan.R) if p != r)) * row / 1e6, 2)
        res[name] = rec
        plan.close()
        del locs, sends, recvs, outs
    return res


def time_tiled(hip, N, stream, base_cfg, steps=3):
    """The tiled path on the same 540x1080 grid with the shape of TERRA Table V's largest model:
    C = 1024 in 8 heads of 128, 32 x 32 windows (1024 tokens; ragged at the grid's edges, 33
    x 17 windows), one SW-MSA module (shift 16, 16) forward and backward, inputs on the device.
    Stage times come from the library's trace events; algorithmic FLOPs as for the chain."""
    import numpy as np
    import torch
    from workloads.configs import SwinConfig
    cfg = SwinConfig(name="w32_hd128", batch=1, grid=base_cfg.grid, channels=1024, heads=8, window=(1, 32, 32),
                     shifts=((0, 16, 16),), dtype="bf16", backward=True, periodic=base_cfg.periodic,
                     description="540x1080, C=1024, 8 heads x 128, 32x32 windows")
    g = torch.Generator(device="cuda")
    g.manual_seed(2)
    C = cfg.channels
    desc = N.make_desc(cfg.batch, cfg.grid, C, cfg.heads, cfg.window, cfg.shifts[0], cfg.periodic, N.SWIN_BF16)
    plan = N.Plan(desc)
    wq = (torch.randn(3 * C, C, device="cuda", generator=g) * (1.0 / (2 * C)) ** 0.5).to(torch.bfloat16)
    wp = (torch.randn(C, C, device="cuda", generator=g) * (1.0 / C) ** 0.5).to(torch.bfloat16)
    tab = torch.randn(cfg.bias_table_shape(), device="cuda", generator=g) * 0.02
    shape = (1,) + tuple(cfg.grid) + (C,)
    x = torch.randn(shape, device="cuda", generator=g).to(torch.bfloat16)
    dy = torch.randn(shape, device="cuda", generator=g).to(torch.bfloat16)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    saved, ws = plan.alloc_saved(), plan.alloc_bwd_ws()
    gw = [torch.empty(3 * C, C, device="cuda"), torch.empty(C, C, device="cuda"), torch.empty_like(tab)]

    def step():
        N.swin_attn_fwd(plan.handle, x, wq, None, wp, None, tab, y, saved, stream=stream)
        N.swin_attn_bwd(plan.handle, dy, x, wq, wp, tab, saved, dx, gw[0], None, gw[1], None, gw[2], ws,
                        stream=stream)

    step()
    torch.cuda.synchronize()
    per = len(FWD_STAGES) + 1 + len(BWD_STAGES) + 1
    ev = hip.events(per * steps)
    N.swin_attn_trace_events(ev)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    assert N.swin_attn_trace_cursor() == per * steps
    N.swin_attn_trace_events(None)
    dur = {st: [] for st in FWD_STAGES + BWD_STAGES}
    k = 0
    for _ in range(steps):
        for stages in (FWD_STAGES, BWD_STAGES):
            for j, st in enumerate(stages):
                dur[st].append(hip.elapsed_ms(ev[k + j], ev[k + j + 1]))
            k += len(stages) + 1
    total = float(sum(np.mean(v) for v in dur.values()))
    hip.destroy(ev)
    f, _ = stage_flops_bytes(cfg, plan.stats["allowed_pairs"])
    core_fwd, core_bwd = f["attn_fwd"], f["attn_bwd"]
    res = {"config": cfg.description, "windows": int(plan.stats["n_windows"]),
           "max_tokens": int(plan.stats["max_tokens"]), "steps": steps, "ms_per_step": round(total, 3),
           "tflops": round(sum(f.values()) / (total * 1e-3) / 1e12, 1),
           "mfma_peak_frac": round(sum(f.values()) / (total * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "attn_fwd_ms": round(float(np.mean(dur["attn_fwd"])), 3),
           "attn_fwd_tflops": round(core_fwd / (np.mean(dur["attn_fwd"]) * 1e-3) / 1e12, 1),
           "attn_bwd_ms": round(float(np.mean(dur["attn_bwd"])), 3),
           "attn_bwd_tflops": round(core_bwd / (np.mean(dur["attn_bwd"]) * 1e-3) / 1e12, 1),
           "stage_ms": {k2: round(float(np.mean(v)), 3) for k2, v in dur.items()}}
    plan.close()
    return res


def time_block_chain(hip, N, stream, cfg, steps, warmup, hidden_mult=4):
    """Two Swin blocks (W-MSA block, then SW-MSA block: layer norms, attention module, GELU MLP of
    hidden width 4C, residuals) forward and backward on the full grid, inputs and weights drawn on
    the device. FLOPs: the attention module's products plus the two MLP products (4 T C H per
    block forward, twice that backward); layer norms, GELU and residual adds are not counted."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    C = cfg.channels
    H = hidden_mult * C
    T = cfg.n_tokens

    def rnd(*shape, scale=1.0, dtype=torch.bfloat16):
        return (torch.randn(*shape, device="cuda", generator=g) * scale).to(dtype)
    blocks = []
    for i, shift in enumerate(cfg.shifts):
        desc = N.make_desc(cfg.batch, cfg.grid, C, cfg.heads, cfg.window, shift, cfg.periodic, N.SWIN_BF16)
        plan = N.BlockPlan(N.make_block_desc(desc, hidden=H))
        prm = {"ln1_g": 1 + rnd(C, scale=0.1), "ln1_b": rnd(C, scale=0.1),
               "w_qkv": rnd(3 * C, C, scale=(2.0 / (4 * C)) ** 0.5), "b_qkv": rnd(3 * C, scale=0.1),
               "w_proj": rnd(C, C, scale=(1.0 / C) ** 0.5), "b_proj": rnd(C, scale=0.1),
               "bias_table": rnd(*cfg.bias_table_shape(), scale=0.02, dtype=torch.float32),
               "ln2_g": 1 + rnd(C, scale=0.1), "ln2_b": rnd(C, scale=0.1),
               "w1": rnd(H, C, scale=(2.0 / (C + H)) ** 0.5), "b1": rnd(H, scale=0.1),
               "w2": rnd(C, H, scale=(2.0 / (C + H)) ** 0.5), "b2": rnd(C, scale=0.1)}
        grads = {k: torch.empty(v.shape, dtype=torch.float32, device="cuda") for k, v in prm.items()}
        blocks.append((plan, prm, grads, plan.alloc_saved(), plan.alloc_bwd_ws()))
    shape = (cfg.batch,) + tuple(cfg.grid) + (C,)
    x = rnd(*shape)
    dy = rnd(*shape)
    y1, y2, dx2, dx1 = (torch.empty_like(x) for _ in range(4))

    def step():
        (p1, w1, g1, s1, ws1), (p2, w2, g2, s2, ws2) = blocks
        N.swin_block_fwd(p1.handle, x, w1, y1, s1, stream=stream)
        N.swin_block_fwd(p2.handle, y1, w2, y2, s2, stream=stream)
        N.swin_block_bwd(p2.handle, dy, y1, w2, s2, dx2, g2, ws2, stream=stream)
        N.swin_block_bwd(p1.handle, dx2, x, w1, s1, dx1, g1, ws1, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = hip.events(2)
    assert hip.l.hipEventRecord(t0, stream.cuda_stream) == 0
    for _ in range(steps):
        step()
    assert hip.l.hipEventRecord(t1, stream.cuda_stream) == 0
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(t0, t1) / steps
    hip.destroy([t0, t1])
    flops = 0
    for plan, *_ in blocks:
        st = N.swin_attn_host_stats(plan.desc.attn)
        f, _ = stage_flops_bytes(cfg, st["allowed_pairs"])
        flops += sum(f.values()) + 3 * 4 * T * C * H
    res = {"hidden": H, "steps": steps, "ms_per_step": round(ms, 4),
           "tokens_per_s": round(T * len(blocks) / (ms * 1e-3), 1), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
           "mfma_peak_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "algorithmic_gflop_per_step": round(flops / 1e9, 2)}
    for plan, *_ in blocks:
        plan.close()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--device-inputs", action="store_true",
                    help="draw inputs on the GPU (torch generator, same shapes and scales) instead of the seeded "
                         "host recipe: starts in seconds, for profiler runs; implies --no-cpu-baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path (the window decomposition "
              "would shard by lat stripes, one rank per GPU, with the token routes exchanging boundary windows); "
              "got --gpus %d" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from __graft_entry__ import _ensure_built
    _ensure_built()
    from shifted_window_attention_amd import native as N
    from shifted_window_attention_amd.device import ModuleOnDevice, to_dev
    from workloads import get_config, make_inputs

    cfg = get_config("highres")
    torch.cuda.set_device(0)
    if args.device_inputs:
        args.no_cpu_baseline = True
        log("bench: drawing inputs on the device", cfg.description)
        inp = _device_inputs(cfg)
        x, dy = inp.x_t, inp.dy_t
    else:
        log("bench: generating inputs", cfg.description)
        inp = make_inputs(cfg, bias_scale=0.0)
        x = to_dev(inp.x_dev, "bf16")
        dy = to_dev(inp.dy_dev, "bf16")
    mods = [ModuleOnDevice(cfg, i, p) for i, p in enumerate(inp.modules)]
    C = cfg.channels
    y1 = torch.empty_like(x)
    y2 = torch.empty_like(x)
    dx2 = torch.empty_like(x)
    dx1 = torch.empty_like(x)
    grads = [{"w_qkv": torch.empty(3 * C, C, dtype=torch.float32, device="cuda"),
              "b_qkv": torch.empty(3 * C, dtype=torch.float32, device="cuda"),
              "w_proj": torch.empty(C, C, dtype=torch.float32, device="cuda"),
              "b_proj": torch.empty(C, dtype=torch.float32, device="cuda"),
              "table": torch.empty_like(m.table)} for m in mods]
    stream = torch.cuda.current_stream()

    def step():
        m1, m2 = mods
        N.swin_attn_fwd(m1.plan.handle, x, m1.w_qkv, m1.b_qkv, m1.w_proj, m1.b_proj, m1.table, y1, m1.saved,
                        stream=stream)
        N.swin_attn_fwd(m2.plan.handle, y1, m2.w_qkv, m2.b_qkv, m2.w_proj, m2.b_proj, m2.table, y2, m2.saved,
                        stream=stream)
        g = grads[1]
        N.swin_attn_bwd(m2.plan.handle, dy, y1, m2.w_qkv, m2.w_proj, m2.table, m2.saved, dx2, g["w_qkv"],
                        g["b_qkv"], g["w_proj"], g["b_proj"], g["table"], m2.ws, stream=stream)
        g = grads[0]
        N.swin_attn_bwd(m1.plan.handle, dx2, x, m1.w_qkv, m1.w_proj, m1.table, m1.saved, dx1, g["w_qkv"],
                        g["b_qkv"], g["w_proj"], g["b_proj"], g["table"], m1.ws, stream=stream)

    log("bench: warmup", args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    hip = Hip()
    # the timed steps: one event at each step boundary and nothing recorded inside a step
    bounds = hip.events(args.steps + 1)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    assert hip.l.hipEventRecord(bounds[0], stream.cuda_stream) == 0
    for i in range(args.steps):
        step()
        assert hip.l.hipEventRecord(bounds[i + 1], stream.cuda_stream) == 0
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = [hip.elapsed_ms(bounds[i], bounds[i + 1]) for i in range(args.steps)]
    total_ms = hip.elapsed_ms(bounds[0], bounds[args.steps])
    ms_step = total_ms / args.steps
    hip.destroy(bounds)

    # per-stage durations from the same number of steps run again with the library's trace
    # events (recorded between stages on the library's stream; each call's events bracket its
    # stages)
    per_step = 2 * (len(FWD_STAGES) + 1) + 2 * (len(BWD_STAGES) + 1)
    ev = hip.events(per_step * args.steps)
    N.swin_attn_trace_events(ev)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    recorded = N.swin_attn_trace_cursor()
    N.swin_attn_trace_events(None)
    assert recorded == per_step * args.steps, (recorded, per_step * args.steps)
    durations = {s: [] for s in FWD_STAGES + BWD_STAGES}
    k = 0
    for _ in range(args.steps):
        for stages in (FWD_STAGES, FWD_STAGES, BWD_STAGES, BWD_STAGES):
            for j, s in enumerate(stages):
                durations[s].append(hip.elapsed_ms(ev[k + j], ev[k + j + 1]))
            k += len(stages) + 1
    hip.destroy(ev)

    pairs = [m.plan.stats["allowed_pairs"] for m in mods]
    flops_step = 0
    bytes_mod = []
    flops_mod = []
    for pr in pairs:
        f, b = stage_flops_bytes(cfg, pr)
        flops_mod.append(f)
        bytes_mod.append(b)
        flops_step += sum(f.values())
    tflops = flops_step / (ms_step * 1e-3) / 1e12
    hbm_bytes_step = sum(sum(b.values()) for b in bytes_mod)
    tokens_step = cfg.n_tokens * cfg.modules
    value = tokens_step / (ms_step * 1e-3)

    kernels = {}
    for s, d in durations.items():
        avg = float(np.mean(d))
        fl = float(np.mean([f[s] for f in flops_mod]))
        by = float(np.mean([b[s] for b in bytes_mod]))
        rec = {"avg_ms": round(avg, 4), "ms_per_step": round(float(np.sum(d)) / args.steps, 4),
               "launches_per_step": len(d) // args.steps}
        if fl:
            rec["tflops"] = round(fl / (avg * 1e-3) / 1e12, 1)
            rec["mfma_frac"] = round(rec["tflops"] / PEAK_BF16_TFLOPS, 4)
        if by:
            rec["gbs"] = round(by / (avg * 1e-3) / 1e9, 1)
            rec["hbm_frac"] = round(rec["gbs"] / PEAK_HBM_GBS, 4)
        kernels[s] = rec
    # dominant single-kernel stage
    dom = max((s for s in kernels if s in STAGE_KERNEL), key=lambda s: kernels[s]["ms_per_step"])
    dk = kernels[dom]
    is_core = dom.startswith("attn")
    dom_flops = float(np.mean([f[dom] for f in flops_mod]))
    dom_bytes = float(np.mean([b[dom] for b in bytes_mod]))
    if is_core:
        roof = {"bound": "hbm", "achieved": dk["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(dk["gbs"] / PEAK_HBM_GBS, 4)}
        per_launch_ref = dom_bytes
    else:
        roof = {"bound": "mfma", "achieved": dk["tflops"], "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                "frac": round(dk["tflops"] / PEAK_BF16_TFLOPS, 4)}
        per_launch_ref = dom_flops
    roof["kernel"] = STAGE_KERNEL[dom][0]
    roof["stage"] = dom
    roof["avg_launch_ms"] = dk["avg_ms"]
    roof["algorithmic_per_launch"] = per_launch_ref
    roof["traffic"] = traffic_for(dom, per_launch_ref)

    moves = time_window_moves(hip, N, mods[1].plan.handle, x, stream, cfg)
    shard = time_shard_share(hip, N, stream, cfg, max(1, args.steps // 2), max(1, args.warmup // 2))
    offload = time_offload(hip, N, stream, mods, x, dy, (y1, y2, dx2, dx1), grads, 3)
    offload["chain_ms_per_step"] = round(ms_step, 4)
    recompute = time_recompute(hip, N, stream, mods, x, dy, (y1, y2, dx2, dx1), grads, max(1, args.steps // 5))
    # the activations of the attention chain are no longer needed: free them before the blocks
    del mods, grads, y1, y2, dx2, dx1
    torch.cuda.empty_cache()
    block = time_block_chain(hip, N, stream, cfg, max(1, args.steps // 5), max(1, args.warmup // 5))
    routes = time_routes(hip, N, stream, cfg)
    tiled = time_tiled(hip, N, stream, cfg)
    configs = {}
    for name in ("om4", "ragged", "levels3d", "tiny"):
        log("bench: workload", name)
        configs[name] = time_config(hip, N, stream, name, calls=max(args.steps, 50), warmup=max(args.warmup, 10),
                                    with_cpu=not args.no_cpu_baseline)
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: oracle CPU baseline (~%.0f s)" % args.cpu_seconds)
        cpu = cpu_baseline(cfg, inp, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "swin W-MSA -> SW-MSA chain fwd+bwd, 540x1080 lat-lon tokens (2160x4320 field after "
                               "4x4 patch embedding), batch 1, C=512, 16 heads x 32, window 12x12, shift (6,6), "
                               "lon periodic, lat masked",
                   "tokens": cfg.n_tokens, "modules": cfg.modules, "global_batch": cfg.batch, "seq_len": 144,
                   "parallelism": "single GPU"},
        "tflops": round(tflops, 1), "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "step_ms": {"median": round(float(np.median(step_ms)), 4), "min": round(float(np.min(step_ms)), 4),
                    "max": round(float(np.max(step_ms)), 4)},
        "hbm_bytes_per_step": int(hbm_bytes_step),
        "algorithmic_gflop_per_step": round(flops_step / 1e9, 2),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "roofline": roof, "kernels": kernels, "window_moves": moves, "shard_share_8way": shard,
        "swin_block_chain": block, "saved_offload": offload, "recompute_qkv": recompute,
        "token_routes_8_ranks": routes, "tiled_w32_hd128": tiled, "configs": configs, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
