"""Device-side helpers over the binding: host arrays to device tensors and back, and the
attention module / Swin block with their plan, device weights, saved state and workspace.

Argument marshalling and buffer ownership only: every step of the method runs in the HIP
library through the C ABI (native.py). Used by bench.py, the smoke check and the GPU tests."""
import numpy as np


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) to float64 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_dev(arr, dtype):
    import torch
    if arr is None:
        return None
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def from_dev(t):
    import torch
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.double().cpu().numpy()


class ModuleOnDevice:
    """One attention module: plan + device weights."""

    def __init__(self, cfg, module_idx, params, with_bias=True):
        import torch
        from shifted_window_attention_amd import native as N
        self.N = N
        self.cfg = cfg
        self.dt = cfg.dtype
        desc = N.make_desc(cfg.batch, cfg.grid, cfg.channels, cfg.heads, cfg.window, cfg.shifts[module_idx],
                           cfg.periodic, N.SWIN_BF16 if cfg.dtype == "bf16" else N.SWIN_F32)
        self.plan = N.Plan(desc)
        self.w_qkv = to_dev(params.w_qkv_dev, self.dt)
        self.b_qkv = to_dev(params.b_qkv_dev, self.dt) if with_bias else None
        self.w_proj = to_dev(params.w_proj_dev, self.dt)
        self.b_proj = to_dev(params.b_proj_dev, self.dt) if with_bias else None
        self.table = torch.from_numpy(np.ascontiguousarray(params.table_dev, dtype=np.float32)).cuda()
        self.saved = self.plan.alloc_saved()
        self.ws = self.plan.alloc_bwd_ws() if cfg.dtype == "bf16" else None
        self.torch = torch

    def fwd(self, x):
        y = self.torch.empty_like(x)
        self.N.swin_attn_fwd(self.plan.handle, x, self.w_qkv, self.b_qkv, self.w_proj, self.b_proj, self.table, y,
                             self.saved)
        return y

    def bwd(self, dy, x):
        t = self.torch
        C = self.cfg.channels
        dx = t.empty_like(dy)
        g = {"w_qkv": t.empty(3 * C, C, dtype=t.float32, device="cuda"),
             "b_qkv": t.empty(3 * C, dtype=t.float32, device="cuda"),
             "w_proj": t.empty(C, C, dtype=t.float32, device="cuda"),
             "b_proj": t.empty(C, dtype=t.float32, device="cuda"),
             "table": t.empty_like(self.table)}
        self.N.swin_attn_bwd(self.plan.handle, dy, x, self.w_qkv, self.w_proj, self.table, self.saved, dx,
                             g["w_qkv"], g["b_qkv"], g["w_proj"], g["b_proj"], g["table"], self.ws)
        return dx, g


def run_chain(cfg, inp, with_bwd=True, with_bias=True):
    """Forward through every chained module, then backward in reverse. Returns numpy (float64) results."""
    import torch
    mods = [ModuleOnDevice(cfg, i, p, with_bias) for i, p in enumerate(inp.modules)]
    x = to_dev(inp.x_dev, cfg.dtype)
    xs = [x]
    for m in mods:
        xs.append(m.fwd(xs[-1]))
    out = {"y": from_dev(xs[-1])}
    if with_bwd:
        d = to_dev(inp.dy_dev, cfg.dtype)
        grads = [None] * len(mods)
        for i in reversed(range(len(mods))):
            d, grads[i] = mods[i].bwd(d, xs[i])
        out["dx"] = from_dev(d)
        out["grads"] = [{k: v.double().cpu().numpy() for k, v in g.items()} for g in grads]
    torch.cuda.synchronize()
    out["mods"] = mods
    out["xs"] = xs
    return out


BLOCK_FIELDS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_proj", "b_proj", "bias_table", "ln2_g", "ln2_b", "w1",
                "b1", "w2", "b2")


class BlockOnDevice:
    """One Swin block: block plan + device parameters (attention module and extras)."""

    def __init__(self, cfg, module_idx, params, extras, hidden=0):
        import torch
        from shifted_window_attention_amd import native as N
        self.N = N
        self.cfg = cfg
        desc = N.make_desc(cfg.batch, cfg.grid, cfg.channels, cfg.heads, cfg.window, cfg.shifts[module_idx],
                           cfg.periodic, N.SWIN_BF16)
        self.plan = N.BlockPlan(N.make_block_desc(desc, hidden=hidden))
        self.H = extras.w1.shape[0]
        p = {"w_qkv": to_dev(params.w_qkv_dev, "bf16"), "b_qkv": to_dev(params.b_qkv_dev, "bf16"),
             "w_proj": to_dev(params.w_proj_dev, "bf16"), "b_proj": to_dev(params.b_proj_dev, "bf16"),
             "bias_table": torch.from_numpy(np.ascontiguousarray(params.table_dev, dtype=np.float32)).cuda()}
        for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b", "w1", "b1", "w2", "b2"):
            p[k] = to_dev(extras.dev[k], "bf16")
        self.params = p
        self.saved = self.plan.alloc_saved()
        self.ws = self.plan.alloc_bwd_ws()
        self.torch = torch

    def fwd(self, x):
        y = self.torch.empty_like(x)
        self.N.swin_block_fwd(self.plan.handle, x, self.params, y, self.saved)
        return y

    def grad_buffers(self):
        t = self.torch
        return {k: t.empty(v.shape, dtype=t.float32, device="cuda") for k, v in self.params.items()}

    def bwd(self, dy, x):
        dx = self.torch.empty_like(dy)
        g = self.grad_buffers()
        self.N.swin_block_bwd(self.plan.handle, dy, x, self.params, self.saved, dx, g, self.ws)
        return dx, g


def run_block_chain(cfg, inp, extras, with_bwd=True):
    """The chained Swin blocks on the device; numpy (float64) results, gradients under the
    oracle's names (bias_table -> table)."""
    import torch
    blocks = [BlockOnDevice(cfg, i, p, e, hidden=e.w1.shape[0]) for i, (p, e) in enumerate(zip(inp.modules, extras))]
    x = to_dev(inp.x_dev, "bf16")
    xs = [x]
    for b in blocks:
        xs.append(b.fwd(xs[-1]))
    out = {"y": from_dev(xs[-1])}
    if with_bwd:
        d = to_dev(inp.dy_dev, "bf16")
        grads = [None] * len(blocks)
        for i in reversed(range(len(blocks))):
            d, g = blocks[i].bwd(d, xs[i])
            g["table"] = g.pop("bias_table")
            grads[i] = g
        out["dx"] = from_dev(d)
        out["grads"] = [{k: v.double().cpu().numpy() for k, v in g.items()} for g in grads]
    torch.cuda.synchronize()
    out["blocks"] = blocks
    out["xs"] = [from_dev(v) for v in xs]
    return out
