"""Oracle-side runners: whole chains of modules or Swin blocks on small grids, and sampled
windows of full-size grids.

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: used by the tests, the smoke check and
the bench's CPU-baseline leg. Only the oracle is called here; these are restrictions of the
full oracle (the same per-window definition evaluated on the windows a check needs)."""
import numpy as np

from . import swin_oracle as O


def params_of(m):
    return O.Params(m.w_qkv, m.b_qkv, m.w_proj, m.b_proj, m.table)


def layouts(cfg):
    return [O.window_layout(cfg.batch, cfg.grid, cfg.window, s, cfg.periodic) for s in cfg.shifts]


def _grad_dict(g):
    d = {"w_qkv": g.w_qkv, "b_qkv": g.b_qkv, "w_proj": g.w_proj, "b_proj": g.b_proj, "table": g.table}
    if g.abs is not None:
        d["abs"] = g.abs
    return d


def chain_full(cfg, inp, with_bwd=True, with_bias=True):
    lays = layouts(cfg)
    ps = [params_of(m) for m in inp.modules]
    if not with_bias:
        for p in ps:
            p.b_qkv = np.zeros_like(p.b_qkv)
            p.b_proj = np.zeros_like(p.b_proj)
    xs = [inp.x]
    lses = []
    for p, lay in zip(ps, lays):
        y, saved = O.module_fwd(xs[-1], p, lay, cfg.heads)
        xs.append(y)
        lses.append(saved["lse"])
    out = {"y": xs[-1], "lse": lses}
    if with_bwd:
        d = inp.dy
        grads = [None] * len(ps)
        for i in reversed(range(len(ps))):
            d, g = O.module_bwd(d, xs[i], ps[i], lays[i], cfg.heads, with_abs=True)
            grads[i] = _grad_dict(g)
        out["dx"] = d
        out["grads"] = grads
    return out


def _windows_of_tokens(lay, tokens):
    """Ids of the windows that hold the given flat grid indices."""
    inv = np.empty_like(lay.perm)
    inv[lay.perm] = np.arange(lay.n_tokens)
    offs = np.array([w.tok_off for w in lay.windows])
    slots = inv[np.asarray(tokens)]
    return sorted(set((np.searchsorted(offs, slots, side="right") - 1).tolist()))


def _tokens_of_windows(lay, wids):
    return np.concatenate([lay.perm[lay.windows[i].tok_off:lay.windows[i].tok_off + lay.windows[i].n]
                           for i in wids])


def chain_sampled(cfg, inp, last_windows, with_bwd=True):
    """Oracle outputs of a 1- or 2-module chain on the tokens of `last_windows` (window ids of
    the last module): y there and, with_bwd, dx at the chain input on the tokens of the first
    module's windows `last_windows` maps back to. Returns flat-index arrays with the values."""
    lays = layouts(cfg)
    ps = [params_of(m) for m in inp.modules]
    C = cfg.channels
    xflat = inp.x.reshape(-1, C)
    res = {}
    if len(lays) == 1:
        lay, p = lays[0], ps[0]
        xw = O.gather(inp.x, lay)
        yw, _ = O.windows_fwd(xw, p, lay, cfg.heads, window_ids=last_windows)
        toks = _tokens_of_windows(lay, last_windows)
        slots = np.concatenate([np.arange(lay.windows[i].tok_off, lay.windows[i].tok_off + lay.windows[i].n)
                                for i in last_windows])
        res["y_tokens"], res["y"] = toks, yw[slots]
        if with_bwd:
            g = O.windows_bwd(O.gather(inp.dy, lay), xw, p, lay, cfg.heads, window_ids=last_windows)
            res["dx_tokens"], res["dx"] = toks, g.dxw[slots]
        return res
    assert len(lays) == 2
    l1, l2 = lays
    p1, p2 = ps
    # forward: y2 on the tokens of S2 needs y1 on those tokens, i.e. module 1 on the windows holding them
    S2 = list(last_windows)
    T2 = _tokens_of_windows(l2, S2)
    S1f = _windows_of_tokens(l1, T2)
    xw1 = O.gather(inp.x, l1)
    y1w, _ = O.windows_fwd(xw1, p1, l1, cfg.heads, window_ids=S1f)
    y1 = np.full_like(xflat, np.nan)
    y1[_tokens_of_windows(l1, S1f)] = y1w[np.concatenate(
        [np.arange(l1.windows[i].tok_off, l1.windows[i].tok_off + l1.windows[i].n) for i in S1f])]
    y1g = y1.reshape(inp.x.shape)
    y2w, _ = O.windows_fwd(O.gather(y1g, l2), p2, l2, cfg.heads, window_ids=S2)
    slots2 = np.concatenate([np.arange(l2.windows[i].tok_off, l2.windows[i].tok_off + l2.windows[i].n) for i in S2])
    res["y_tokens"], res["y"] = T2, y2w[slots2]
    if not with_bwd:
        return res
    # backward: dx1 on the tokens of a module-1 window set S1 needs dy1 (= dx2) on those tokens,
    # i.e. module 2's backward on the windows holding them, which needs y1 on their tokens.
    S1 = _windows_of_tokens(l1, T2)[:max(1, len(S2))]
    T1 = _tokens_of_windows(l1, S1)
    S2b = _windows_of_tokens(l2, T1)
    T2b = _tokens_of_windows(l2, S2b)
    S1fb = _windows_of_tokens(l1, T2b)
    y1b = np.full_like(xflat, np.nan)
    y1bw, _ = O.windows_fwd(xw1, p1, l1, cfg.heads, window_ids=S1fb)
    y1b[_tokens_of_windows(l1, S1fb)] = y1bw[np.concatenate(
        [np.arange(l1.windows[i].tok_off, l1.windows[i].tok_off + l1.windows[i].n) for i in S1fb])]
    g2 = O.windows_bwd(O.gather(inp.dy, l2), O.gather(y1b.reshape(inp.x.shape), l2), p2, l2, cfg.heads,
                       window_ids=S2b)
    dx2 = np.full_like(xflat, np.nan)
    slots2b = np.concatenate([np.arange(l2.windows[i].tok_off, l2.windows[i].tok_off + l2.windows[i].n)
                              for i in S2b])
    dx2[T2b] = g2.dxw[slots2b]
    g1 = O.windows_bwd(O.gather(dx2.reshape(inp.x.shape), l1), xw1, p1, l1, cfg.heads, window_ids=S1)
    slots1 = np.concatenate([np.arange(l1.windows[i].tok_off, l1.windows[i].tok_off + l1.windows[i].n) for i in S1])
    res["dx_tokens"], res["dx"] = T1, g1.dxw[slots1]
    return res


def chain_masked_dy(cfg, inp, last_windows, dy_masked):
    """Oracle gradients when dy is zero outside the tokens of `last_windows` (windows of the
    last module): every reduction then only sums over the windows it reaches, which are
    computed here in full. Returns dx (flat tokens + values) and the per-module gradients."""
    lays = layouts(cfg)
    ps = [params_of(m) for m in inp.modules]
    C = cfg.channels
    shape = inp.x.shape
    res = {"grads": [None] * len(lays)}
    if len(lays) == 1:
        lay, p = lays[0], ps[0]
        g = O.windows_bwd(O.gather(dy_masked, lay), O.gather(inp.x, lay), p, lay, cfg.heads,
                          window_ids=last_windows, with_abs=True)
        res["grads"][0] = _grad_dict(g)
        toks = _tokens_of_windows(lay, last_windows)
        slots = np.concatenate([np.arange(lay.windows[i].tok_off, lay.windows[i].tok_off + lay.windows[i].n)
                                for i in last_windows])
        res["dx_tokens"], res["dx"] = toks, g.dxw[slots]
        return res
    l1, l2 = lays
    p1, p2 = ps
    S2 = list(last_windows)
    T2 = _tokens_of_windows(l2, S2)
    S1f = _windows_of_tokens(l1, T2)
    xw1 = O.gather(inp.x, l1)
    y1w, _ = O.windows_fwd(xw1, p1, l1, cfg.heads, window_ids=S1f)
    y1 = np.full((inp.x.reshape(-1, C).shape[0], C), np.nan)
    slots1f = np.concatenate([np.arange(l1.windows[i].tok_off, l1.windows[i].tok_off + l1.windows[i].n)
                              for i in S1f])
    y1[_tokens_of_windows(l1, S1f)] = y1w[slots1f]
    g2 = O.windows_bwd(O.gather(dy_masked, l2), O.gather(y1.reshape(shape), l2), p2, l2, cfg.heads,
                       window_ids=S2, with_abs=True)
    res["grads"][1] = _grad_dict(g2)
    dy1 = np.zeros_like(y1)
    slots2 = np.concatenate([np.arange(l2.windows[i].tok_off, l2.windows[i].tok_off + l2.windows[i].n) for i in S2])
    dy1[T2] = g2.dxw[slots2]
    g1 = O.windows_bwd(O.gather(dy1.reshape(shape), l1), xw1, p1, l1, cfg.heads, window_ids=S1f, with_abs=True)
    res["grads"][0] = _grad_dict(g1)
    res["dx_tokens"], res["dx"] = _tokens_of_windows(l1, S1f), g1.dxw[slots1f]
    return res


def block_params_of(m, e):
    """Oracle parameters of one Swin block: attention module m, extras e (layer norms, MLP)."""
    from . import block_oracle as BO
    return BO.BlockParams(ln1_g=e.ln1_g, ln1_b=e.ln1_b, attn=params_of(m), ln2_g=e.ln2_g, ln2_b=e.ln2_b,
                          w1=e.w1, b1=e.b1, w2=e.w2, b2=e.b2)


def block_chain_full(cfg, inp, extras, with_bwd=True):
    """The chained Swin blocks (one per shift of cfg) forward, then backward in reverse."""
    from . import block_oracle as BO
    lays = layouts(cfg)
    ps = [block_params_of(m, e) for m, e in zip(inp.modules, extras)]
    xs = [inp.x]
    for p, lay in zip(ps, lays):
        y, _ = BO.block_fwd(xs[-1], p, lay, cfg.heads)
        xs.append(y)
    out = {"y": xs[-1], "xs": xs}
    if with_bwd:
        d = inp.dy
        grads = [None] * len(ps)
        for i in reversed(range(len(ps))):
            g = BO.block_bwd(d, xs[i], ps[i], lays[i], cfg.heads)
            d = g.pop("dx")
            grads[i] = g
        out["dx"] = d
        out["grads"] = grads
    return out
