"""fp64 CPU oracle for shifted-window multi-head self-attention (W-MSA / SW-MSA).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import or call
this module: only the tests, the smoke check and the bench's CPU-baseline leg
use it. It shares no code with the HIP library.

What it computes, and from which passage:

* Token grid: a channels-last B x H x W x C field on a regular lat-lon grid
  (TERRA page, section II-A), generalised to B x D x H x W x C with vertical
  levels.
* Shift: between attention layers the whole domain is rolled by half a
  window in both spatial dimensions (BEAST page, "Model Architecture" and
  "Domain-Tensor Parallelism"). Reading: roll by -s, i.e. the rolled field is
  x~[i'] = x[(i' + s) mod N] on every axis.
* Partition: a token at (u, v) belongs to window (u div w, v div w) at
  within-window offset (u mod w, v mod w) (TERRA page, section IV-D); the
  window grid is flattened in row-major order and indexed 0..M-1 (TERRA page,
  section V-A, Eq. 4). Reading for grids that do not divide evenly: the last
  window along an axis is short and is attended without padding.
* W-MSA / SW-MSA (TERRA page, section IV-A and Fig. 4: Block 0 W-MSA,
  Block 1 SW-MSA; BEAST page, "Domain-Tensor Parallelism": a QKV map, then
  attention independently per head, then head concatenation). The pages never
  write the attention formula; reading: standard Swin attention
  softmax(tau * q k^T + T[rel] + mask) v with tau = head_dim^-1/2, the
  relative-position bias added after scaling, and -inf between tokens whose
  wrap labels differ on a non-periodic axis.
* Reverse: the inverse permutation returns every token to its grid position
  (TERRA page, section IV-D: routes restore tokens at their destination
  positions and their backward passes apply the inverse mappings).

Every function works in float64 on values that the caller has already rounded
to the run dtype. Pins that check this module against things other than
itself live in tests/test_oracle_*.py.
"""
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# Index maps: roll -> partition -> labels (steps 1-3)
# ---------------------------------------------------------------------------


@dataclass
class Window:
    b: int
    k: Tuple[int, int, int]        # window index along (D, H, W)
    start: Tuple[int, int, int]    # first rolled-frame index along each axis
    ext: Tuple[int, int, int]      # extents (short for the last window of a ragged axis)
    tok_off: int                   # first window-major token slot
    n: int                         # tokens in the window


@dataclass
class Layout:
    batch: int
    grid: Tuple[int, int, int]
    window: Tuple[int, int, int]
    shift: Tuple[int, int, int]
    periodic: int
    perm: np.ndarray        # [N_tok] int64: window-major slot -> flat grid index (b,d,h,w row-major)
    labels: np.ndarray      # [N_tok] uint8 bit mask: bit a = wrap label on axis a
    local: np.ndarray       # [N_tok, 3] int64 within-window offsets (ld, lh, lw)
    windows: List[Window]

    @property
    def n_tokens(self) -> int:
        return int(self.perm.shape[0])


def axis_labels(N: int, s: int, periodic: bool) -> np.ndarray:
    """Wrap label of every rolled-frame index along one axis.

    After rolling by -s the last s rolled indices hold tokens that came from
    the start of the axis. On a non-periodic axis those tokens are not
    neighbours of the ones before them, so they carry label 1 (reading of the
    shift-region mask); on a periodic axis, or with no shift, every label is 0.
    """
    lab = np.zeros(N, dtype=np.uint8)
    if not periodic and s > 0:
        lab[N - s:] = 1
    return lab


def window_layout(batch: int, grid: Sequence[int], window: Sequence[int],
                  shift: Sequence[int], periodic: int) -> Layout:
    """Literal roll + row-major partition of the token grid (steps 1-3)."""
    D, H, W = (int(g) for g in grid)
    wd, wh, ww = (int(w) for w in window)
    sd, sh, sw = (int(s) for s in shift)
    idx = np.arange(batch * D * H * W, dtype=np.int64).reshape(batch, D, H, W)
    # step 1: roll by -s; np.roll(a, -s)[i'] == a[(i' + s) mod N]
    rolled = np.roll(idx, shift=(-sd, -sh, -sw), axis=(1, 2, 3))
    labs = [axis_labels(N, s, bool(periodic >> a & 1)) for a, (N, s) in enumerate(((D, sd), (H, sh), (W, sw)))]
    perm, labels, local, windows = [], [], [], []
    off = 0
    nk = [(N + w - 1) // w for N, w in ((D, wd), (H, wh), (W, ww))]
    for b in range(batch):
        for kd in range(nk[0]):
            for kh in range(nk[1]):
                for kw in range(nk[2]):
                    d0, h0, w0 = kd * wd, kh * wh, kw * ww
                    d1, h1, w1 = min(d0 + wd, D), min(h0 + wh, H), min(w0 + ww, W)
                    block = rolled[b, d0:d1, h0:h1, w0:w1]
                    ext = block.shape
                    n = block.size
                    perm.append(block.reshape(-1))
                    ld, lh, lw = np.meshgrid(np.arange(ext[0]), np.arange(ext[1]), np.arange(ext[2]), indexing="ij")
                    local.append(np.stack([ld.ravel(), lh.ravel(), lw.ravel()], axis=1))
                    lab = (labs[0][d0:d1][:, None, None] * 1 + labs[1][h0:h1][None, :, None] * 2
                           + labs[2][w0:w1][None, None, :] * 4)
                    labels.append(lab.astype(np.uint8).reshape(-1))
                    windows.append(Window(b=b, k=(kd, kh, kw), start=(d0, h0, w0), ext=tuple(ext),
                                          tok_off=off, n=n))
                    off += n
    return Layout(batch=batch, grid=(D, H, W), window=(wd, wh, ww), shift=(sd, sh, sw), periodic=periodic,
                  perm=np.concatenate(perm), labels=np.concatenate(labels), local=np.concatenate(local),
                  windows=windows)


def gather(x: np.ndarray, layout: Layout) -> np.ndarray:
    """Grid [B, D, H, W, C] -> window-major token rows [N_tok, C]."""
    C = x.shape[-1]
    return x.reshape(-1, C)[layout.perm]


def scatter(xw: np.ndarray, layout: Layout) -> np.ndarray:
    """Window-major token rows -> grid (step 9: inverse permutation)."""
    C = xw.shape[-1]
    out = np.empty_like(xw)
    out[layout.perm] = xw
    D, H, W = layout.grid
    return out.reshape(layout.batch, D, H, W, C)


def roll_unroll_grid(x: np.ndarray, layout: Layout) -> np.ndarray:
    """Step 9 written as the literal inverse of steps 1-2: undo the partition, then roll by +s."""
    B, D, H, W, C = x.shape
    xr = np.roll(x, shift=tuple(-s for s in layout.shift), axis=(1, 2, 3))
    back = np.empty_like(xr)
    xw = gather(x, layout)
    for win in layout.windows:
        d0, h0, w0 = win.start
        ed, eh, ew = win.ext
        back[win.b, d0:d0 + ed, h0:h0 + eh, w0:w0 + ew] = xw[win.tok_off:win.tok_off + win.n].reshape(ed, eh, ew, C)
    assert np.array_equal(back, xr)
    return np.roll(back, shift=layout.shift, axis=(1, 2, 3))


# ---------------------------------------------------------------------------
# Relative-position bins (reading: query minus key, offset by w-1, row-major table)
# ---------------------------------------------------------------------------


def rel_bins(local_q: np.ndarray, local_k: np.ndarray, window: Sequence[int]) -> np.ndarray:
    """Flat index into a [2wd-1, 2wh-1, 2ww-1] table for every (query, key) pair."""
    wd, wh, ww = window
    d = local_q[:, None, :] - local_k[None, :, :] + np.array([wd - 1, wh - 1, ww - 1])
    return (d[..., 0] * (2 * wh - 1) + d[..., 1]) * (2 * ww - 1) + d[..., 2]


# ---------------------------------------------------------------------------
# Forward (steps 4-8) and backward on window-major rows
# ---------------------------------------------------------------------------


@dataclass
class Params:
    w_qkv: np.ndarray  # [3C, C]
    b_qkv: np.ndarray  # [3C]
    w_proj: np.ndarray  # [C, C]
    b_proj: np.ndarray  # [C]
    table: np.ndarray   # [nh, 2wd-1, 2wh-1, 2ww-1]


def _groups(layout: Layout, window_ids: Optional[Sequence[int]], max_batch: int):
    """Windows grouped by extent (same token count), in chunks of max_batch."""
    ids = range(len(layout.windows)) if window_ids is None else window_ids
    by_ext: Dict[Tuple[int, int, int], List[int]] = {}
    for i in ids:
        by_ext.setdefault(layout.windows[i].ext, []).append(i)
    for ext, lst in by_ext.items():
        for c in range(0, len(lst), max_batch):
            yield ext, lst[c:c + max_batch]


def _window_rows(layout: Layout, wids: Sequence[int]) -> np.ndarray:
    return np.stack([np.arange(layout.windows[i].tok_off, layout.windows[i].tok_off + layout.windows[i].n)
                     for i in wids])


def _bias_and_mask(layout: Layout, rows: np.ndarray, table_h: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Logit offsets for one group: bias [nh, n, n] (same for every window of an extent) and
    allowed [G, n, n] (labels equal on every axis)."""
    loc = layout.local[rows[0]]
    bins = rel_bins(loc, loc, layout.window)                      # [n, n]
    bias = table_h.reshape(table_h.shape[0], -1)[:, bins]          # [nh, n, n]
    lab = layout.labels[rows]                                      # [G, n]
    allowed = lab[:, :, None] == lab[:, None, :]
    return bias, allowed, bins


def windows_fwd(xw: np.ndarray, p: Params, layout: Layout, heads: int, scale: Optional[float] = None,
                window_ids: Optional[Sequence[int]] = None, max_batch: int = 64, keep: bool = False):
    """Attention module on window-major rows. Returns yw (rows outside window_ids are NaN)
    and, if keep, a dict of per-group intermediates (P, LSE, q, k, v, o)."""
    N, C = xw.shape
    hd = C // heads
    tau = hd ** -0.5 if not scale else scale
    yw = np.full((N, C), np.nan)
    saved = {"lse": np.full((N, heads), np.nan), "o": np.full((N, C), np.nan), "groups": []}
    for ext, wids in _groups(layout, window_ids, max_batch):
        rows = _window_rows(layout, wids)                          # [G, n]
        G, n = rows.shape
        xt = xw[rows]                                              # [G, n, C]
        qkv = xt @ p.w_qkv.T + p.b_qkv                             # step 4
        q = qkv[..., 0 * C:1 * C].reshape(G, n, heads, hd).transpose(0, 2, 1, 3)
        k = qkv[..., 1 * C:2 * C].reshape(G, n, heads, hd).transpose(0, 2, 1, 3)
        v = qkv[..., 2 * C:3 * C].reshape(G, n, heads, hd).transpose(0, 2, 1, 3)
        bias, allowed, _ = _bias_and_mask(layout, rows, p.table)
        s = tau * (q @ k.transpose(0, 1, 3, 2)) + bias[None]       # step 5
        s = np.where(allowed[:, None], s, -np.inf)
        m = s.max(axis=-1, keepdims=True)                          # step 6
        e = np.exp(s - m)
        z = e.sum(axis=-1, keepdims=True)
        P = e / z
        lse = (m + np.log(z))[..., 0]                              # [G, nh, n]
        o = (P @ v).transpose(0, 2, 1, 3).reshape(G, n, C)         # step 7
        yt = o @ p.w_proj.T + p.b_proj                             # step 8
        yw[rows] = yt
        saved["lse"][rows] = lse.transpose(0, 2, 1)
        saved["o"][rows] = o
        if keep:
            saved["groups"].append({"rows": rows, "P": P, "q": q, "k": k, "v": v, "allowed": allowed})
    return yw, saved


@dataclass
class Grads:
    dxw: np.ndarray
    w_qkv: np.ndarray
    b_qkv: np.ndarray
    w_proj: np.ndarray
    b_proj: np.ndarray
    table: np.ndarray
    # with_abs: for every reduced gradient, the same sum taken over the absolute values of its
    # terms (e.g. sum_t |d(qkv)_t|^T |x~_t| for dW_qkv, sum of |dS| per bin for dT). A
    # diagnostic that leaves the gradients unchanged: it measures how much the terms cancel,
    # which sets how far rounding in the terms can move the sum.
    abs: Optional[Dict[str, np.ndarray]] = None


def windows_bwd(dyw: np.ndarray, xw: np.ndarray, p: Params, layout: Layout, heads: int,
                scale: Optional[float] = None, window_ids: Optional[Sequence[int]] = None,
                max_batch: int = 64, with_abs: bool = False) -> Grads:
    """Hand-derived backward of windows_fwd (forward recomputed per group).

    dW_proj = dy~^T o; db_proj = sum dy~; do = dy~ W_proj;
    dv = P^T do; dP = do v^T; D = rowsum(P * dP); dS = P * (dP - D);
    dq = tau dS k; dk = tau dS^T q; dT[h, bin] = sum of dS over windows and allowed pairs;
    dW_qkv = d(qkv)^T x~; db_qkv = sum d(qkv); dx~ = d(qkv) W_qkv.
    Reductions cover only the windows in window_ids (all by default)."""
    N, C = xw.shape
    hd = C // heads
    tau = hd ** -0.5 if not scale else scale
    g = Grads(dxw=np.full((N, C), np.nan), w_qkv=np.zeros_like(p.w_qkv), b_qkv=np.zeros_like(p.b_qkv),
              w_proj=np.zeros_like(p.w_proj), b_proj=np.zeros_like(p.b_proj), table=np.zeros_like(p.table))
    nbins = p.table[0].size
    dtab = g.table.reshape(heads, nbins)
    if with_abs:
        g.abs = {k: np.zeros_like(getattr(g, k)) for k in ("w_qkv", "b_qkv", "w_proj", "b_proj", "table")}
        atab = g.abs["table"].reshape(heads, nbins)
    for ext, wids in _groups(layout, window_ids, max_batch):
        rows = _window_rows(layout, wids)
        G, n = rows.shape
        xt = xw[rows]
        qkv = xt @ p.w_qkv.T + p.b_qkv
        q = qkv[..., 0 * C:1 * C].reshape(G, n, heads, hd).transpose(0, 2, 1, 3)
        k = qkv[..., 1 * C:2 * C].reshape(G, n, heads, hd).transpose(0, 2, 1, 3)
        v = qkv[..., 2 * C:3 * C].reshape(G, n, heads, hd).transpose(0, 2, 1, 3)
        bias, allowed, bins = _bias_and_mask(layout, rows, p.table)
        s = tau * (q @ k.transpose(0, 1, 3, 2)) + bias[None]
        s = np.where(allowed[:, None], s, -np.inf)
        m = s.max(axis=-1, keepdims=True)
        e = np.exp(s - m)
        P = e / e.sum(axis=-1, keepdims=True)
        o = (P @ v).transpose(0, 2, 1, 3).reshape(G, n, C)
        dyt = dyw[rows]                                            # [G, n, C]
        g.w_proj += np.einsum("gnc,gnd->cd", dyt, o)
        g.b_proj += dyt.sum(axis=(0, 1))
        if with_abs:
            g.abs["w_proj"] += np.einsum("gnc,gnd->cd", np.abs(dyt), np.abs(o))
            g.abs["b_proj"] += np.abs(dyt).sum(axis=(0, 1))
        do = (dyt @ p.w_proj).reshape(G, n, heads, hd).transpose(0, 2, 1, 3)
        dv = P.transpose(0, 1, 3, 2) @ do
        dP = do @ v.transpose(0, 1, 3, 2)
        Dr = (P * dP).sum(axis=-1, keepdims=True)
        dS = P * (dP - Dr)                                         # zero on masked pairs (P == 0)
        dq = tau * (dS @ k)
        dk = tau * (dS.transpose(0, 1, 3, 2) @ q)
        dsum = dS.sum(axis=0)                                      # [nh, n, n]
        for h in range(heads):
            np.add.at(dtab[h], bins.ravel(), dsum[h].ravel())
        if with_abs:
            asum = np.abs(dS).sum(axis=0)
            for h in range(heads):
                np.add.at(atab[h], bins.ravel(), asum[h].ravel())
        dqkv = np.concatenate([t.transpose(0, 2, 1, 3).reshape(G, n, C) for t in (dq, dk, dv)], axis=-1)
        g.w_qkv += np.einsum("gnc,gnd->cd", dqkv, xt)
        g.b_qkv += dqkv.sum(axis=(0, 1))
        if with_abs:
            g.abs["w_qkv"] += np.einsum("gnc,gnd->cd", np.abs(dqkv), np.abs(xt))
            g.abs["b_qkv"] += np.abs(dqkv).sum(axis=(0, 1))
        g.dxw[rows] = dqkv @ p.w_qkv
    return g


# ---------------------------------------------------------------------------
# Whole module on the grid
# ---------------------------------------------------------------------------


def module_fwd(x: np.ndarray, p: Params, layout: Layout, heads: int, scale: Optional[float] = None,
               max_batch: int = 64):
    xw = gather(x, layout)
    yw, saved = windows_fwd(xw, p, layout, heads, scale, max_batch=max_batch)
    return scatter(yw, layout), saved


def module_bwd(dy: np.ndarray, x: np.ndarray, p: Params, layout: Layout, heads: int,
               scale: Optional[float] = None, max_batch: int = 64, with_abs: bool = False):
    """Returns (dx on the grid, Grads with dxw)."""
    g = windows_bwd(gather(dy, layout), gather(x, layout), p, layout, heads, scale, max_batch=max_batch,
                    with_abs=with_abs)
    return scatter(g.dxw, layout), g


# ---------------------------------------------------------------------------
# Brute force: an independent per-token formulation for tiny grids
# ---------------------------------------------------------------------------


def brute_force_fwd(x: np.ndarray, p: Params, grid: Sequence[int], window: Sequence[int], shift: Sequence[int],
                    periodic: int, heads: int, scale: Optional[float] = None) -> np.ndarray:
    """For every original token: compute its rolled coordinates, window and labels directly from
    (t, s, w); collect its keys by scanning every token of the grid; form logits with explicit loops
    and softmax with a Python loop. No roll, reshape or partition is used."""
    B, D, H, W, C = x.shape
    N = (D, H, W)
    hd = C // heads
    tau = hd ** -0.5 if not scale else scale
    wts = p.table.reshape(heads, -1)
    tab_dims = tuple(2 * w - 1 for w in window)

    def coords(d, h, w):
        out = []
        for a, i in enumerate((d, h, w)):
            r = (i - shift[a]) % N[a]                # rolled index: x~[r] = x[(r + s) mod N]
            lab = 1 if (not (periodic >> a & 1) and shift[a] > 0 and r + shift[a] >= N[a]) else 0
            out.append((r // window[a], r % window[a], lab))
        return out

    tokens = [(b, d, h, w) for b in range(B) for d in range(D) for h in range(H) for w in range(W)]
    info = {t: coords(*t[1:]) for t in tokens}
    qkv = {t: p.w_qkv @ x[t] + p.b_qkv for t in tokens}
    y = np.zeros_like(x)
    for t in tokens:
        ci = info[t]
        keys = [u for u in tokens if u[0] == t[0] and all(
            info[u][a][0] == ci[a][0] and info[u][a][2] == ci[a][2] for a in range(3))]
        o = np.zeros(C)
        for h in range(heads):
            qh = qkv[t][h * hd:(h + 1) * hd]
            logits = []
            for u in keys:
                kh = qkv[u][C + h * hd:C + (h + 1) * hd]
                rel = [ci[a][1] - info[u][a][1] + window[a] - 1 for a in range(3)]
                b_idx = (rel[0] * tab_dims[1] + rel[1]) * tab_dims[2] + rel[2]
                logits.append(tau * float(np.dot(qh, kh)) + wts[h, b_idx])
            mx = max(logits)
            ex = [np.exp(l - mx) for l in logits]
            z = sum(ex)
            for wgt, u in zip(ex, keys):
                o[h * hd:(h + 1) * hd] += (wgt / z) * qkv[u][2 * C + h * hd:2 * C + (h + 1) * hd]
        y[t] = p.w_proj @ o + p.b_proj
    return y


# ---------------------------------------------------------------------------
# Second formulation of a mask-split window: unmasked sub-windows
# ---------------------------------------------------------------------------


def windows_fwd_split(xw: np.ndarray, p: Params, layout: Layout, heads: int, scale: Optional[float] = None):
    """Forward in which every window is cut into its label groups and each group is attended as an
    unmasked sub-window (no -inf anywhere). Equal to windows_fwd if the mask reading is right."""
    N, C = xw.shape
    hd = C // heads
    tau = hd ** -0.5 if not scale else scale
    yw = np.empty((N, C))
    tab = p.table.reshape(heads, -1)
    for win in layout.windows:
        rows = np.arange(win.tok_off, win.tok_off + win.n)
        for lab in np.unique(layout.labels[rows]):
            sub = rows[layout.labels[rows] == lab]
            xt = xw[sub]
            qkv = xt @ p.w_qkv.T + p.b_qkv
            loc = layout.local[sub]
            bins = rel_bins(loc, loc, layout.window)
            o = np.empty((len(sub), C))
            for h in range(heads):
                q = qkv[:, h * hd:(h + 1) * hd]
                k = qkv[:, C + h * hd:C + (h + 1) * hd]
                v = qkv[:, 2 * C + h * hd:2 * C + (h + 1) * hd]
                s = tau * q @ k.T + tab[h][bins]
                s = s - s.max(axis=1, keepdims=True)
                e = np.exp(s)
                o[:, h * hd:(h + 1) * hd] = (e / e.sum(axis=1, keepdims=True)) @ v
            yw[sub] = o @ p.w_proj.T + p.b_proj
    return yw


# ---------------------------------------------------------------------------
# Algorithmic work (what the method itself must compute)
# ---------------------------------------------------------------------------


def allowed_pairs(layout: Layout) -> int:
    """Number of (query, key) pairs with equal labels, summed over all windows."""
    total = 0
    for win in layout.windows:
        lab = layout.labels[win.tok_off:win.tok_off + win.n]
        cnt = np.bincount(lab, minlength=8).astype(np.int64)
        total += int((cnt * cnt).sum())
    return total


def module_flops(n_tokens: int, channels: int, heads: int, pairs: int) -> Dict[str, int]:
    """Forward FLOPs of one module: QKV GEMM, proj GEMM and the two attention products over
    allowed pairs; backward is twice the forward (recomputation not counted)."""
    hd = channels // heads
    qkv = 2 * n_tokens * channels * 3 * channels
    proj = 2 * n_tokens * channels * channels
    core = 4 * hd * pairs * heads
    fwd = qkv + proj + core
    return {"qkv": qkv, "proj": proj, "core": core, "fwd": fwd, "bwd": 2 * fwd, "fwd_bwd": 3 * fwd}
