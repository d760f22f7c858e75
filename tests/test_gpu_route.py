"""Token routes on the device (include/swin_route.h): pack, loopback exchange and restore,
bit-exact against the route oracle's placement of every token, for the DMP route (stripes ->
unshifted windows), the shift route (unshifted -> shifted windows) and their inverses, on
small grids and on the 540x1080, C=512 grid over 8 ranks."""
import numpy as np
import pytest

from oracle import route_oracle as RO
from tests.gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from shifted_window_attention_amd import native  # noqa: F401  (raises if the library is missing)


def _coded(n_tok, words):
    """Row g, 16-bit word c holds (g * 31 + c) mod 2^16: every row is distinct."""
    g = np.arange(n_tok, dtype=np.int64)[:, None]
    c = np.arange(words, dtype=np.int64)[None, :]
    return ((g * 31 + c) % 65536 - 32768).astype(np.int16)


def _oracle_layout(batch, grid, win, per, kind, ranks, shift):
    if kind == 0:
        return RO.stripes_layout(batch, grid, ranks)
    return RO.windows_layout(batch, grid, win, shift, per, ranks)


def _route_on_device(N, gdesc, src, dst, locals_dev, words):
    import torch
    plan = N.RoutePlan(gdesc, N.make_rank_layout(*src), N.make_rank_layout(*dst))
    assert [t.shape[0] for t in locals_dev] == plan.src_sizes.tolist()
    sends = [torch.empty((int(n), words), dtype=torch.int16, device="cuda") for n in plan.src_sizes]
    recvs = [torch.empty((int(n), words), dtype=torch.int16, device="cuda") for n in plan.dst_sizes]
    outs = [torch.full((int(n), words), -1, dtype=torch.int16, device="cuda") for n in plan.dst_sizes]
    for p in range(plan.P):
        N.swin_route_pack(plan, p, locals_dev[p], sends[p])
    N.swin_route_loopback(plan, sends, recvs)
    for r in range(plan.R):
        N.swin_route_unpack(plan, r, recvs[r], outs[r])
    torch.cuda.synchronize()
    counts = plan.counts.copy()
    plan.close()
    return outs, counts


def _run_case(batch, grid, win, per, C, layouts):
    """Route the coded grid through the chain of layouts; compare every stage with the oracle."""
    import torch
    from shifted_window_attention_amd import native as N
    n_tok = batch * grid[0] * grid[1] * grid[2]
    words = C  # bf16 rows: C 16-bit words
    x = _coded(n_tok, words)
    gdesc = N.make_desc(batch, grid, C, 1, win, (0, 0, 0), per, N.SWIN_BF16)
    lays = [_oracle_layout(batch, grid, win, per, *l) for l in layouts]
    cur = [torch.from_numpy(a).cuda() for a in RO.distribute(x.reshape((batch,) + tuple(grid) + (words,)), lays[0])]
    for i in range(1, len(layouts)):
        cur, counts = _route_on_device(N, gdesc, layouts[i - 1], layouts[i], cur, words)
        want = RO.distribute(x.reshape((batch,) + tuple(grid) + (words,)), lays[i])
        for r, (a, b) in enumerate(zip(cur, want)):
            assert np.array_equal(a.cpu().numpy(), b), (i, r)
        log("  stage %d: %s -> %s, tokens moved between ranks %d of %d" % (
            i, layouts[i - 1][:2], layouts[i][:2], int(counts.sum() - np.trace(counts)) if counts.shape[0] ==
            counts.shape[1] else -1, n_tok))


SMALL = [
    (1, (1, 24, 36), (1, 6, 6), 4, 64, 3, 4),     # lon periodic, P != R
    (1, (1, 25, 37), (1, 6, 8), 4, 64, 4, 5),     # ragged edge windows
    (2, (3, 10, 12), (2, 4, 4), 0, 192, 2, 6),    # batch 2, 3-D, C = 192
    (1, (1, 12, 12), (1, 6, 6), 6, 64, 3, 7),     # more window ranks than windows
]


@pytest.mark.parametrize("batch,grid,win,per,C,P,R", SMALL)
def test_routes_small(batch, grid, win, per, C, P, R):
    log("routes", batch, grid, win, "P", P, "R", R)
    sh = tuple(w // 2 for w in win)
    _run_case(batch, grid, win, per, C, [(0, P, (0, 0, 0)), (1, R, (0, 0, 0)), (1, R, sh), (1, R, (0, 0, 0)),
                                         (0, P, (0, 0, 0))])


def test_routes_full_size_8_ranks():
    """540x1080 tokens, C = 512, 12x12 windows, 8 stripes -> 8 window ranks, shift (6, 6), and back."""
    log("routes 540x1080 C=512 over 8 ranks")
    _run_case(1, (1, 540, 1080), (1, 12, 12), 4, 512,
              [(0, 8, (0, 0, 0)), (1, 8, (0, 0, 0)), (1, 8, (0, 6, 6)), (1, 8, (0, 0, 0)), (0, 8, (0, 0, 0))])


def test_route_device_errors():
    import torch
    from shifted_window_attention_amd import native as N
    gdesc = N.make_desc(1, (1, 24, 36), 64, 1, (1, 6, 6), (0, 0, 0), 4, N.SWIN_BF16)
    plan = N.RoutePlan(gdesc, N.make_rank_layout(0, 3), N.make_rank_layout(1, 4))
    buf = torch.zeros((int(plan.src_sizes[0]), 64), dtype=torch.int16, device="cuda")
    for fn in (lambda: N.swin_route_pack(plan, 3, buf, torch.empty_like(buf)),      # rank out of range
               lambda: N.swin_route_pack(plan, 0, buf, buf),                        # aliasing
               lambda: N.swin_route_unpack(plan, -1, buf, torch.empty_like(buf)),
               lambda: N.swin_route_loopback(plan, [None, None, None], [None] * 4)):
        with pytest.raises(N.SwinError) as e:
            fn()
        assert e.value.status == 1
    torch.cuda.synchronize()
    plan.close()
