"""The saved-state offload engine (include/swin_offload.h) through the C ABI: byte-exact round
trips through pinned host memory, ordering after the producing stream, a backward run on a
saved state that went to the host and back (bitwise equal to the one that stayed), ticket
reuse, and argument errors."""
import numpy as np
import pytest

from tests.gpu_util import ModuleOnDevice, log, to_dev
from workloads import get_config, make_inputs
from workloads.configs import small_variant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from shifted_window_attention_amd import native  # noqa: F401  (raises if the library is missing)


@pytest.fixture()
def engine():
    from shifted_window_attention_amd import native as N
    e = N.swin_offload_create(0)
    yield e
    N.swin_offload_destroy(e)


def test_round_trip_is_byte_exact(engine):
    import torch
    from shifted_window_attention_amd import native as N
    n = (3 << 20) + 123                      # not a multiple of any copy granule
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    dev = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=g)
    ref = dev.cpu().numpy().copy()
    host = N.PinnedBuffer(n)
    t1 = N.swin_offload_store(engine, dev, host, n)
    N.swin_offload_sync(engine)
    assert N.swin_offload_query(engine, t1)
    assert np.array_equal(host.array, ref)
    stream = torch.cuda.current_stream()
    N.swin_offload_wait(engine, t1, stream)  # the store has read dev: now it may be overwritten
    dev.zero_()
    t2 = N.swin_offload_load(engine, host, dev, n, after=stream)
    assert t2 == t1 + 1
    N.swin_offload_wait(engine, t2, stream)
    assert np.array_equal(dev.cpu().numpy(), ref)
    assert N.swin_offload_bytes(engine) == (n, n)
    host.free()


def test_store_is_ordered_after_the_producer(engine):
    """A store issued right after a fill on the caller's stream sees the filled values."""
    import torch
    from shifted_window_attention_amd import native as N
    n = 64 << 20
    dev = torch.zeros(n, dtype=torch.uint8, device="cuda")
    host = N.PinnedBuffer(n)
    stream = torch.cuda.current_stream()
    for value in (7, 19, 201):
        dev.fill_(value)                        # enqueued, not finished
        t = N.swin_offload_store(engine, dev, host, n, after=stream)
        N.swin_offload_wait(engine, t, stream)  # the next fill must not overtake the copy
        N.swin_offload_sync(engine)
        assert int(host.array.min()) == value and int(host.array.max()) == value
    host.free()


def test_backward_after_offload_matches_resident(engine):
    import torch
    from shifted_window_attention_amd import native as N
    cfg = small_variant(get_config("highres"), grid=(1, 36, 48))
    inp = make_inputs(cfg)
    log("offload round trip of the saved state,", cfg.grid)
    m0 = ModuleOnDevice(cfg, 0, inp.modules[0])
    m1 = ModuleOnDevice(cfg, 1, inp.modules[1])
    x = to_dev(inp.x_dev, "bf16")
    dy = to_dev(inp.dy_dev, "bf16")
    stream = torch.cuda.current_stream()
    # resident reference
    y0 = m0.fwd(x)
    dx_ref, g_ref = m0.bwd(dy, x)
    torch.cuda.synchronize()
    # offload: forward, store the saved state, let another module run, wipe, load, backward
    nbytes = m0.plan.saved_bytes
    host = N.PinnedBuffer(nbytes)
    y0b = m0.fwd(x)
    ts = N.swin_offload_store(engine, m0.saved, host, nbytes, after=stream)
    y1 = m1.fwd(y0b)                            # overlaps the copy
    N.swin_offload_wait(engine, ts, stream)
    m0.saved.fill_(0xA5)                        # the device copy is gone
    tl = N.swin_offload_load(engine, host, m0.saved, nbytes, after=stream)
    N.swin_offload_wait(engine, tl, stream)
    dx, g = m0.bwd(dy, x)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y0b.view(torch.int16))
    assert torch.equal(dx.view(torch.int16), dx_ref.view(torch.int16))
    for k in g:
        assert torch.equal(g[k], g_ref[k]), k
    del y1
    host.free()


def test_ticket_ring_reuse():
    import torch
    from shifted_window_attention_amd import native as N
    e = N.swin_offload_create(2)
    n = 1 << 20
    dev = torch.arange(n, dtype=torch.int32, device="cuda").view(torch.uint8)[:n]
    hosts = [N.PinnedBuffer(n) for _ in range(5)]
    tickets = [N.swin_offload_store(e, dev, h, n) for h in hosts]
    assert tickets == [1, 2, 3, 4, 5]
    # tickets 1..3 had their slots reused: complete without any wait
    for t in tickets[:3]:
        assert N.swin_offload_query(e, t)
        N.swin_offload_wait(e, t, torch.cuda.current_stream())
    N.swin_offload_sync(e)
    ref = dev.cpu().numpy()
    for h in hosts:
        assert np.array_equal(h.array, ref)
        h.free()
    N.swin_offload_destroy(e)


def test_argument_errors(engine):
    import torch
    from shifted_window_attention_amd import native as N
    dev = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    host = N.PinnedBuffer(4096)
    pageable = np.zeros(4096, dtype=np.uint8)

    def status(fn):
        with pytest.raises(N.SwinError) as e:
            fn()
        return e.value.status
    assert status(lambda: N.swin_offload_store(engine, dev, host, 0)) == 1
    assert status(lambda: N.swin_offload_store(engine, dev, pageable.ctypes.data, 4096)) == 1
    assert status(lambda: N.swin_offload_store(engine, host, host, 4096)) == 1   # source is not device memory
    assert status(lambda: N.swin_offload_load(engine, dev, dev, 4096)) == 1      # source is not pinned host memory
    assert status(lambda: N.swin_offload_wait(engine, 0)) == 1
    assert status(lambda: N.swin_offload_query(engine, 99)) == 1
    assert status(lambda: N.swin_offload_create(5000)) == 1
    t = N.swin_offload_store(engine, dev, host, 4096)
    N.swin_offload_sync(engine)
    assert N.swin_offload_query(engine, t)
    host.free()
