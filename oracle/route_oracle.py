"""CPU oracle for TERRA's token routes between rank layouts (integer index work, plain NumPy).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import or call this module: only
the tests use it. It shares no code with the HIP library; the window
partition it builds on is the attention oracle's window_layout (oracle/swin_oracle.py).

What it computes, and from which passage (TERRA page):

* Section IV-D: a token is named by its global grid coordinate. Under the DMP stripe layout
  that coordinate fixes the token's source rank and its offset in the rank's spatial stripe;
  under a window assignment it fixes the rank that owns the token's whole window and the
  token's offset in that rank's window-major tensor. Tokens bound for one destination are
  packed into one contiguous send buffer (the index_select step), the buffers are exchanged
  peer to peer, and each destination restores the tokens at their offsets. The shift route is
  the same mechanism between the unshifted and the shifted window partitions; the backward of
  either route is the inverse mapping.
* Section V-A, Eq. 4 (ragged assignment): after flattening the window grid in row-major
  order, rank r of R owns the contiguous window range [floor(r M / R), floor((r + 1) M / R)).

Readings where the page is silent (listed in the design notes as well):

* The DMP stripes split the latitude rows the same way Eq. 4 splits windows: source rank p
  of P owns rows [floor(p H / P), floor((p + 1) H / P)) of every batch element and level,
  stored as a grid-order [B, D, H_p, W] tensor.
* Windows are the attention module's windows, ragged ones included (the page pads the field
  so that all windows are complete; here the short edge windows are windows of their own), in
  the module's row-major order over (batch, level, lat, lon).
* Inside the send buffer of source p the segment for destination r comes before that for
  r + 1, and a segment lists its tokens in destination-offset order; the receive buffer of
  destination r is the concatenation of the segments (p -> r) over p in rank order.
"""
from dataclasses import dataclass
from typing import List, Sequence

import numpy as np

from . import swin_oracle as O


def eq4_ranges(M: int, R: int):
    """TERRA section V-A, Eq. 4: [L_r, R_r) for r = 0..R-1 over M row-major windows."""
    L = [(r * M) // R for r in range(R)]
    Rr = [((r + 1) * M) // R for r in range(R)]
    return L, Rr


@dataclass
class RankLayout:
    """Where every token lives: rank[g] and offset[g] for flat grid index g (b, d, h, w
    row-major), and the number of tokens each rank holds."""
    ranks: int
    rank: np.ndarray      # [N_tok] int64
    offset: np.ndarray    # [N_tok] int64
    sizes: List[int]


def stripes_layout(batch: int, grid: Sequence[int], P: int) -> RankLayout:
    """DMP stripes over latitude (reading above): grid-order local tensors [B, D, H_p, W]."""
    D, H, W = (int(g) for g in grid)
    lo, hi = eq4_ranges(H, P)
    b, d, h, w = np.meshgrid(np.arange(batch), np.arange(D), np.arange(H), np.arange(W), indexing="ij")
    b, d, h, w = (a.reshape(-1) for a in (b, d, h, w))
    rank = np.empty(b.size, dtype=np.int64)
    offset = np.empty(b.size, dtype=np.int64)
    sizes = []
    for p in range(P):
        rows = hi[p] - lo[p]
        sel = (h >= lo[p]) & (h < hi[p])
        rank[sel] = p
        offset[sel] = ((b[sel] * D + d[sel]) * rows + (h[sel] - lo[p])) * W + w[sel]
        sizes.append(batch * D * rows * W)
    return RankLayout(P, rank, offset, sizes)


def windows_layout(batch: int, grid: Sequence[int], window: Sequence[int], shift: Sequence[int], periodic: int,
                   R: int) -> RankLayout:
    """Window assignment of Eq. 4 over the (shifted) window partition: rank r holds its windows'
    tokens window-major, in the module's window order."""
    lay = O.window_layout(batch, grid, window, shift, periodic)
    M = len(lay.windows)
    lo, hi = eq4_ranges(M, R)
    n_tok = lay.perm.size
    starts = [w.tok_off for w in lay.windows] + [n_tok]
    rank = np.empty(n_tok, dtype=np.int64)
    offset = np.empty(n_tok, dtype=np.int64)
    sizes = []
    for r in range(R):
        s0, s1 = starts[lo[r]], starts[hi[r]]
        toks = lay.perm[s0:s1]
        rank[toks] = r
        offset[toks] = np.arange(s1 - s0)
        sizes.append(s1 - s0)
    return RankLayout(R, rank, offset, sizes)


@dataclass
class Route:
    """Index tables of a route from layout src to layout dst."""
    counts: np.ndarray              # [P, R] tokens sent from p to r
    send_src: List[np.ndarray]      # per source p: local source offsets, in send-buffer order
    recv_dst: List[np.ndarray]      # per destination r: local destination offsets, in receive order


def route(src: RankLayout, dst: RankLayout) -> Route:
    P, R = src.ranks, dst.ranks
    counts = np.zeros((P, R), dtype=np.int64)
    seg = {}
    for p in range(P):
        for r in range(R):
            toks = np.nonzero((src.rank == p) & (dst.rank == r))[0]
            toks = toks[np.argsort(dst.offset[toks], kind="stable")]   # destination-offset order
            seg[p, r] = toks
            counts[p, r] = toks.size
    send_src = [np.concatenate([src.offset[seg[p, r]] for r in range(R)]) for p in range(P)]
    recv_dst = [np.concatenate([dst.offset[seg[p, r]] for p in range(P)]) for r in range(R)]
    return Route(counts, send_src, recv_dst)


def distribute(x: np.ndarray, lay: RankLayout) -> List[np.ndarray]:
    """Per-rank local tensors [size_r, C] of a global grid tensor [B, D, H, W, C]."""
    C = x.shape[-1]
    flat = x.reshape(-1, C)
    out = [np.zeros((n, C), dtype=x.dtype) for n in lay.sizes]
    for r in range(lay.ranks):
        sel = np.nonzero(lay.rank == r)[0]
        out[r][lay.offset[sel]] = flat[sel]
    return out


def pack(local: np.ndarray, rt: Route, p: int) -> np.ndarray:
    """Send buffer of source p: its tokens for every destination, segment after segment."""
    return local[rt.send_src[p]]


def exchange(sends: List[np.ndarray], rt: Route) -> List[np.ndarray]:
    """The peer-to-peer step: destination r receives segment (p -> r) of every source p."""
    P, R = rt.counts.shape
    offs = np.concatenate([np.zeros((P, 1), dtype=np.int64), np.cumsum(rt.counts, axis=1)], axis=1)
    return [np.concatenate([sends[p][offs[p, r]:offs[p, r + 1]] for p in range(P)]) for r in range(R)]


def unpack(recv: np.ndarray, rt: Route, r: int, size: int) -> np.ndarray:
    """Destination r restores every received token at its local offset."""
    out = np.zeros((size,) + recv.shape[1:], dtype=recv.dtype)
    out[rt.recv_dst[r]] = recv
    return out


def apply_route(locals_: List[np.ndarray], src: RankLayout, dst: RankLayout) -> List[np.ndarray]:
    """pack -> exchange -> unpack, every rank in one process (loopback)."""
    rt = route(src, dst)
    sends = [pack(locals_[p], rt, p) for p in range(src.ranks)]
    recvs = exchange(sends, rt)
    return [unpack(recvs[r], rt, r, dst.sizes[r]) for r in range(dst.ranks)]
