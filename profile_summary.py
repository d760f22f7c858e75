"""Short text summaries of rocprofv3 runs of bench.py, for profiles/.

  python profile_summary.py trace DIR OUT.md --cmd "<rocprofv3 command>"
      per-kernel table from the --kernel-trace --stats CSV (kernel_stats.csv) under DIR
  python profile_summary.py counters DIR [DIR ...] --cmd "<rocprofv3 command, {counters} for the list>"
      per-stage SQ counters from --pmc runs (each DIR one pass of at most 8 SQ counters plus
      GRBM_GUI_ACTIVE), with the derived MFMA, VALU, LDS and wait figures, written to
      profiles/counters_540x1080_c512.md
  python profile_summary.py traffic FETCH_DIR WRITE_DIR --cmd-fetch "..." --cmd-write "..."
      HBM bytes per dispatch from two --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per
      dispatch), each scaled by what the same counter reads for the window gather, a copy of
      known size (n_tok x C bf16 rows plus the int32 permutation in, the rows out). Writes
      profiles/traffic.json (read by bench.py for its roofline "traffic" field) and
      profiles/traffic_540x1080_c512.md.

Kernels launched more than once per step with different shapes (the two GEMM kernels) are
told apart by their position in the step's fixed launch order: within the attention chain
(every dispatch before the first stand-alone window move, which bench.py times after the chain) and
within the Swin-block chain (from the first layer-norm dispatch on).
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# launch order of the GEMM kernels within one bench step (W fwd, SW fwd, SW bwd, W bwd); the
# QKV product and dproj (head_dim 32) run on the wide kernel's two instances
NT_ROLES = ["proj_gemm", "proj_gemm", "dgrad_qkv", "dgrad_qkv"]
TN_ROLES = ["wgrad_proj", "wgrad_qkv", "wgrad_proj", "wgrad_qkv"]
SINGLE = {"k_attn_fwd": "attn_fwd", "k_attn_bwd": "attn_bwd", "k_gemm_nt_wide<false>": "qkv_gemm",
          "k_gemm_nt_wide<true>": "dproj_gemm"}
# the same for one step of the two-block chain (block 0 fwd, block 1 fwd, block 1 bwd, block 0 bwd)
NT_BLOCK_ROLES = (["proj_res_gemm", "mlp_w1_gelu", "mlp_w2_res"] * 2 +
                  ["mlp_dgelu", "mlp_dxn", "dgrad_qkv"] * 2)
TN_BLOCK_ROLES = ["wgrad_w2", "wgrad_w1", "wgrad_proj", "wgrad_qkv"] * 2
BLOCK_START = "k_layernorm_fwd"
SOURCES = {"k_gemm_nt": "gemm.hip", "k_gemm_nt_wide": "gemm.hip", "k_gemm_tn": "gemm.hip", "k_attn_fwd": "attn_fwd.hip",
           "k_attn_bwd": "attn_bwd.hip"}
COPY = "k_window_move<true>"


def short(name):
    """Kernel name without return type, namespace and arguments. rocprofv3 leaves some template
    instances mangled (_ZN4swin15k_layernorm_fwdILi1E...): those become the plain name plus
    "<...>", so that base() gives the kernel's name for both spellings."""
    m = re.match(r"_ZN4swin(\d+)", name)
    if m:
        ln = int(m.group(1))
        ident = name[m.end():m.end() + ln]
        rest = name[m.end() + ln:]
        if not rest.startswith("I"):
            return ident
        args, i = [], 1
        while i < len(rest) and rest[i] != "E":  # integer literals and the two element types used here
            lit = re.match(r"Li(\d+)E", rest[i:])
            if lit:
                args.append(lit.group(1))
                i += lit.end()
            elif rest.startswith("Lb0E", i) or rest.startswith("Lb1E", i):
                args.append("true" if rest[i + 2] == "1" else "false")
                i += 4
            elif rest.startswith("DF16b", i):
                args.append("bf16")
                i += 5
            elif rest[i] == "f":
                args.append("float")
                i += 1
            else:
                args.append("?")
                break
        return "%s<%s>" % (ident, ", ".join(args))
    n = name.split("(")[0].replace("void ", "").replace("swin::", "")
    return n.strip()


def base(name):
    return short(name).split("<")[0]


def single_role(name):
    """The stage of a kernel that serves one stage: by its instance, else by its name."""
    return SINGLE.get(short(name)) or SINGLE.get(base(name))


def find(dirname, suffix):
    hits = sorted(glob.glob(os.path.join(dirname, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit("no *%s under %s" % (suffix, dirname))
    return hits[0]


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


def cmd_trace(a):
    path = find(a.dir, "kernel_stats.csv")
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["# Kernel time: %s" % a.title, "", "Command (from the repository root on the GPU host):", "",
             "    " + a.cmd, "", "rocprofv3 kernel_stats, all dispatches of the run (warmup, timed steps and the",
             "stand-alone gather/scatter timing):", "",
             "| kernel | calls | avg us | min us | max us | total ms | % |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| %s | %s | %.1f | %.1f | %.1f | %.2f | %.1f |" % (
            short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    bj = None
    if a.bench_json and os.path.exists(a.bench_json):
        txt = open(a.bench_json).read().strip().splitlines()
        bj = json.loads(txt[-1]) if txt else None
    roles = trace_roles(find(a.dir, "kernel_trace.csv"))
    chain_avg = {}
    for phase, title in (("chain", "attention chain (W-MSA -> SW-MSA modules), every dispatch incl. warmup"),
                         ("block", "Swin-block chain (W-MSA block -> SW-MSA block, MLP 4C), incl. warmup"),
                         ("after", "token-route pack/restore and tiled-path attention kernels (their own "
                                   "measurements), incl. warmup")):
        keys = [k for k in roles if k[0] == phase]
        if not keys:
            continue
        lines += ["", "Per stage, %s (kernel_trace.csv, labelled by launch order):" % title, "",
                  "| stage | dispatches | avg us | min us | max us |", "|---|---|---|---|---|"]
        for k in sorted(keys, key=lambda k: -sum(roles[k])):
            v = roles[k]
            if phase == "chain":
                chain_avg[k[1]] = sum(v) / len(v) / 1e6
            lines.append("| %s | %d | %.1f | %.1f | %.1f |" % (k[1], len(v), sum(v) / len(v) / 1e3, min(v) / 1e3,
                                                               max(v) / 1e3))
    if bj:
        b = bj
        lines += ["", "bench.py line of the same run: %.3f ms/step, %.1f TFLOP/s (%.1f%% of bf16 MFMA peak)" % (
            b["ms_per_step"], b["tflops"], 100 * b["mfma_peak_frac"]), "",
            "| stage | avg ms per launch (bench.py stage events) | avg ms per dispatch (trace, all chain steps) |",
            "|---|---|---|"]
        for k, v in b["kernels"].items():
            t = chain_avg.get(k)
            lines.append("| %s | %.4f | %s |" % (k, v["avg_ms"], "%.4f" % t if t is not None else "-"))
        if b.get("swin_block_chain"):
            bc = b["swin_block_chain"]
            lines += ["", "Swin-block chain: %.3f ms/step, %.1f TFLOP/s (%.1f%% of bf16 MFMA peak)" % (
                bc["ms_per_step"], bc["tflops"], 100 * bc["mfma_peak_frac"])]
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("wrote", a.out)


def trace_roles(path):
    """Per-dispatch durations from kernel_trace.csv, labelled by phase and role:
    {("chain" | "block", role): [ns, ...]} in dispatch order."""
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    out = defaultdict(list)
    phase, seq = "chain", defaultdict(int)
    for r in rows:
        b = base(r["Kernel_Name"])
        if phase == "chain" and b == "k_window_move":
            phase = "moves"
        if phase not in ("block", "after") and b == BLOCK_START:
            phase, seq = "block", defaultdict(int)
        elif phase == "block" and (b == "k_window_move" or b.startswith("k_tiled")):
            phase = "after"  # the route and tiled-path measurements that bench.py runs next
        if phase == "moves" or (phase == "after" and not (b == "k_window_move" or b.startswith("k_tiled"))):
            continue
        ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if b == "k_gemm_nt":
            roles = NT_ROLES if phase == "chain" else NT_BLOCK_ROLES
            role = roles[seq[b] % len(roles)]
        elif b == "k_gemm_tn":
            roles = TN_ROLES if phase == "chain" else TN_BLOCK_ROLES
            role = roles[seq[b] % len(roles)]
        else:
            role = single_role(r["Kernel_Name"]) or short(r["Kernel_Name"])
        seq[b] += 1
        out[(phase, role)].append(ns)
    return out


def per_dispatch(path, counter):
    """{(kernel short name, role): [values]} in dispatch order, for the attention chain (every
    dispatch before the first stand-alone window move) and for the calibration copy (the
    window moves that bench.py times right after the chain, up to the next GEMM)."""
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    out = defaultdict(list)
    seq = defaultdict(int)
    phase = "chain"
    for r in rows:
        name = short(r["Kernel_Name"])
        b = base(r["Kernel_Name"])
        if phase == "chain" and b == "k_window_move":
            phase = "moves"
        elif phase == "moves" and b not in ("k_window_move",) and b.startswith("k_"):
            phase = "rest"
        if phase == "rest":
            break
        v = float(r["Counter_Value"])
        role = None
        if phase == "chain":
            if b == "k_gemm_nt":
                role = NT_ROLES[seq[b] % len(NT_ROLES)]
            elif b == "k_gemm_tn":
                role = TN_ROLES[seq[b] % len(TN_ROLES)]
            elif single_role(r["Kernel_Name"]):
                role = single_role(r["Kernel_Name"])
            seq[b] += 1
        elif name == COPY:
            role = "copy"
        if role:
            out[(name, role)].append(v)
    return out


def cmd_traffic(a):
    from bench import stage_flops_bytes
    from workloads import get_config
    cfg = get_config("highres")
    n, C = cfg.n_tokens, cfg.channels
    fetch = per_dispatch(find(a.fetch_dir, "counter_collection.csv"), "FETCH_SIZE")
    write = per_dispatch(find(a.write_dir, "counter_collection.csv"), "WRITE_SIZE")
    mean = lambda v: sum(v) / len(v)
    cf = [v for (k, r), v in fetch.items() if r == "copy"]
    cw = [v for (k, r), v in write.items() if r == "copy"]
    if not cf or not cw:
        raise SystemExit("no %s dispatches in the counter runs" % COPY)
    copy_read, copy_write = n * C * 2 + n * 4, n * C * 2
    f_read = mean(cf[0]) * 1024 / copy_read
    f_write = mean(cw[0]) * 1024 / copy_write
    # algorithmic bytes of the SW-MSA module (both modules move the same bytes)
    _, alg = stage_flops_bytes(cfg, 0)
    out = {"_calibration": {"copy_kernel": COPY, "copy_read_bytes": copy_read, "copy_write_bytes": copy_write,
                            "fetch_kib": round(mean(cf[0]), 1), "write_kib": round(mean(cw[0]), 1),
                            "fetch_factor": round(f_read, 4), "write_factor": round(f_write, 4)},
           "_commands": {"fetch": a.cmd_fetch, "write": a.cmd_write}}
    lines = ["# HBM traffic per dispatch: 540x1080 tokens, C=512, 16 heads, 12x12 windows", "",
             "Counter runs (from the repository root on the GPU host):", "", "    " + a.cmd_fetch,
             "    " + a.cmd_write, "",
             "Calibration: the window gather (%s) moves a known %d bytes in (rows + int32 permutation) and %d out." %
             (COPY, copy_read, copy_write),
             "FETCH_SIZE reads %.1f KiB for it (factor %.4f), WRITE_SIZE %.1f KiB (factor %.4f); each kernel's counter" %
             (mean(cf[0]), f_read, mean(cw[0]), f_write),
             "is divided by its factor.", "",
             "| stage | kernel | dispatches | FETCH KiB | WRITE KiB | HBM bytes (calibrated) | algorithmic bytes | ratio |",
             "|---|---|---|---|---|---|---|---|"]
    for (kname, role), fv in sorted(fetch.items(), key=lambda t: t[0][1]):
        if role == "copy":
            continue
        wv = write.get((kname, role))
        if not wv:
            continue
        fb = mean(fv) * 1024 / f_read
        wb = mean(wv) * 1024 / f_write
        total = fb + wb
        ab = alg.get(role, 0)
        out[role] = {"kernel": kname, "source_sha": source_sha(SOURCES[base(kname)]), "dispatches": len(fv),
                     "fetch_kib": round(mean(fv), 1), "write_kib": round(mean(wv), 1),
                     "read_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(total),
                     "algorithmic_bytes_per_launch": ab}
        lines.append("| %s | %s | %d | %.0f | %.0f | %.3e | %.3e | %.2f |" % (
            role, kname, len(fv), mean(fv), mean(wv), total, ab, total / ab if ab else float("nan")))
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    json.dump(out, open(os.path.join(ROOT, "profiles", "traffic.json"), "w"), indent=1)
    open(os.path.join(ROOT, "profiles", "traffic_540x1080_c512.md"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


# FLOP per MFMA instruction: the GEMMs run v_mfma_f32_32x32x16_bf16, the attention kernels
# v_mfma_f32_16x16x32_bf16
MFMA_FLOP = {"k_gemm_nt": 2 * 32 * 32 * 16, "k_gemm_nt_wide": 2 * 32 * 32 * 16, "k_gemm_tn": 2 * 32 * 32 * 16, "k_attn_fwd": 2 * 16 * 16 * 32,
             "k_attn_bwd": 2 * 16 * 16 * 32}
N_CU, N_SIMD, N_XCD = 256, 1024, 8


def per_dispatch_rows(path):
    """{counter: {(kernel, role): [(value, ns)]}} for the attention chain, as per_dispatch."""
    rows = list(csv.DictReader(open(path)))
    out = {}
    for c in sorted({r["Counter_Name"] for r in rows}):
        vals = per_dispatch(path, c)
        durs = per_dispatch_durations(path, c)
        out[c] = {k: list(zip(v, durs[k])) for k, v in vals.items()}
    return out


def per_dispatch_durations(path, counter):
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    # same selection and labelling as per_dispatch, with the dispatch duration as the value
    tmp = path + ".dur.csv"
    with open(tmp, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0].keys()))
        w.writeheader()
        for r in rows:
            r = dict(r)
            r["Counter_Value"] = str(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
            w.writerow(r)
    try:
        return per_dispatch(tmp, counter)
    finally:
        os.remove(tmp)


def cmd_counters(a):
    from bench import stage_flops_bytes
    from shifted_window_attention_amd import native as N
    from workloads import get_config
    cfg = get_config("highres")
    pairs = [N.swin_attn_host_stats(N.make_desc(cfg.batch, cfg.grid, cfg.channels, cfg.heads, cfg.window, sh,
                                                cfg.periodic, N.SWIN_BF16))["allowed_pairs"] for sh in cfg.shifts]
    alg = [stage_flops_bytes(cfg, p)[0] for p in pairs]
    data = defaultdict(dict)   # (kernel, role) -> counter -> mean value
    dur = defaultdict(list)
    for d in a.dirs:
        for c, per in per_dispatch_rows(find(d, "counter_collection.csv")).items():
            for k, v in per.items():
                if k[1] == "copy":
                    continue
                data[k][c] = sum(x for x, _ in v) / len(v)
                dur[k] += [ns for _, ns in v]
    mean = lambda v: sum(v) / len(v)
    lines = ["# SQ counters per dispatch: 540x1080 tokens, C=512, 16 heads, 12x12 windows (W-MSA -> SW-MSA fwd+bwd)",
             "", "Counter runs (from the repository root on the GPU host), one per counter set:", ""]
    lines += ["    " + c for c in a.cmd]
    lines += ["", "Every value is the mean over the chain's dispatches of that stage (both modules, warmup and",
              "timed steps), summed over the chip by rocprofv3. Derived figures (cycles = GRBM_GUI_ACTIVE / %d," % N_XCD,
              "the busy cycles of one XCD's command processor over the dispatch):",
              "- MFMA GFLOP = SQ_INSTS_MFMA x FLOP per instruction (32x32x16: 32768, 16x16x32: 16384), against the",
              "  algorithmic GFLOP of the stage (mean of the two modules; the attention kernels also multiply padding",
              "  rows of the last 32-key chunk and form the softmax row sums on the matrix cores);",
              "- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (%d SIMDs x cycles);" % N_SIMD,
              "- VALU busy = 4 x SQ_ACTIVE_INST_VALU / (%d SIMDs x cycles) (a wave64 VALU instruction holds a" % N_SIMD,
              "  16-lane SIMD for 4 cycles; MFMA issue included);",
              "- LDS active = SQ_ACTIVE_INST_LDS / (%d CUs x cycles); bank conflicts = SQ_LDS_BANK_CONFLICT /" % N_CU,
              "  SQ_ACTIVE_INST_LDS;",
              "- waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES (share of resident wave time spent in s_waitcnt).", "",
              "| stage | kernel | us | clock GHz | MFMA GFLOP | alg. GFLOP | MFMA busy | VALU busy | LDS active | "
              "bank confl. | waiting |", "|---|---|---|---|---|---|---|---|---|---|---|"]
    order = ["qkv_gemm", "attn_fwd", "proj_gemm", "dproj_gemm", "wgrad_proj", "attn_bwd", "dgrad_qkv", "wgrad_qkv"]
    for (kname, role) in sorted(data, key=lambda k: order.index(k[1]) if k[1] in order else 99):
        c = data[(kname, role)]
        us = mean(dur[(kname, role)]) / 1e3
        cyc = c.get("GRBM_GUI_ACTIVE", float("nan")) / N_XCD
        f = lambda n: c.get(n, float("nan"))
        mf = f("SQ_INSTS_MFMA") * MFMA_FLOP.get(base(kname), float("nan")) / 1e9
        ag = mean([x.get(role, 0) for x in alg]) / 1e9
        lines.append("| %s | %s | %.0f | %.2f | %.1f | %.1f | %.1f%% | %.1f%% | %.1f%% | %.2f | %.1f%% |" % (
            role, kname, us, cyc / (us * 1e3), mf, ag, 100 * f("SQ_VALU_MFMA_BUSY_CYCLES") / (N_SIMD * cyc),
            100 * 4 * f("SQ_ACTIVE_INST_VALU") / (N_SIMD * cyc), 100 * f("SQ_ACTIVE_INST_LDS") / (N_CU * cyc),
            f("SQ_LDS_BANK_CONFLICT") / f("SQ_ACTIVE_INST_LDS"), 100 * f("SQ_WAIT_ANY") / f("SQ_WAVE_CYCLES")))
    lines += ["", "Raw means per dispatch:", "", "| stage | " + " | ".join(sorted({n for v in data.values() for n in v}))
              + " |", "|---|" + "---|" * len({n for v in data.values() for n in v})]
    names = sorted({n for v in data.values() for n in v})
    for (kname, role) in sorted(data, key=lambda k: order.index(k[1]) if k[1] in order else 99):
        lines.append("| %s | " % role + " | ".join("%.4g" % data[(kname, role)].get(n, float("nan")) for n in names)
                     + " |")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    out = os.path.join(ROOT, "profiles", "counters_540x1080_c512.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("out")
    t.add_argument("--cmd", required=True)
    t.add_argument("--title", default="bench.py, 540x1080 tokens, C=512, W-MSA -> SW-MSA fwd+bwd")
    t.add_argument("--bench-json", default=None)
    f = sub.add_parser("traffic")
    f.add_argument("fetch_dir")
    f.add_argument("write_dir")
    f.add_argument("--cmd-fetch", required=True)
    f.add_argument("--cmd-write", required=True)
    k = sub.add_parser("counters")
    k.add_argument("dirs", nargs="+")
    k.add_argument("--cmd", action="append", required=True)
    a = ap.parse_args()
    {"trace": cmd_trace, "traffic": cmd_traffic, "counters": cmd_counters}[a.what](a)


if __name__ == "__main__":
    main()
