"""The C-ABI library loads, exports every declared symbol, and its host-side
window layout is bit-exact against the oracle (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import swin_oracle as O
from workloads import get_config
from workloads.configs import ORDER

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


@pytest.fixture(scope="module")
def native():
    from shifted_window_attention_amd import native
    return native


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(swin_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_entry_points():
    names = declared_functions()
    for must in ("swin_attn_fwd", "swin_attn_bwd", "swin_window_gather", "swin_window_scatter",
                 "swin_attn_plan_create", "swin_attn_plan_destroy", "swin_attn_sizes", "swin_status_string",
                 "swin_block_plan_create", "swin_block_plan_destroy", "swin_block_sizes", "swin_block_fwd",
                 "swin_block_bwd"):
        assert must in names


def test_block_plan_rejects_unsupported_descriptors(native):
    """Block descriptor checks that run before any device work: fp32, a hidden width that is not a
    multiple of 64, more than 1024 channels and a negative epsilon are refused with a status."""
    cfg = get_config(ORDER[0])
    base = _desc(native, cfg, dtype="bf16")
    bad = [(native.make_block_desc(_desc(native, cfg, dtype="f32")), 2),
           (native.make_block_desc(base, hidden=96), 2),
           (native.make_block_desc(base, ln_eps=-1.0), 1)]
    wide = _desc(native, cfg, dtype="bf16")
    wide.channels = 1088
    wide.heads = 17
    bad.append((native.make_block_desc(wide), 2))
    for d, want in bad:
        h = ctypes.c_void_p()
        st = native.lib.swin_block_plan_create(ctypes.byref(d), ctypes.byref(h))
        assert st == want, (st, native.lib.swin_attn_last_error())
        assert not h.value


def test_library_exports_every_declared_symbol(native):
    raw = ctypes.CDLL(native.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def _desc(native, cfg, module=0, dtype=None):
    return native.make_desc(cfg.batch, cfg.grid, cfg.channels, cfg.heads, cfg.window, cfg.shifts[module],
                            cfg.periodic, native.SWIN_BF16 if (dtype or cfg.dtype) == "bf16" else native.SWIN_F32)


CASES = [(n, m) for n in ORDER for m in range(get_config(n).modules)]


@pytest.mark.parametrize("name,module", CASES)
def test_host_index_map_bit_exact(native, name, module):
    cfg = get_config(name)
    lay = O.window_layout(cfg.batch, cfg.grid, cfg.window, cfg.shifts[module], cfg.periodic)
    m, lab = native.swin_attn_host_index_map(_desc(native, cfg, module))
    assert np.array_equal(m, lay.perm)
    assert np.array_equal(lab, lay.labels)


@pytest.mark.parametrize("name,module", CASES)
def test_host_stats_match_oracle(native, name, module):
    cfg = get_config(name)
    lay = O.window_layout(cfg.batch, cfg.grid, cfg.window, cfg.shifts[module], cfg.periodic)
    st = native.swin_attn_host_stats(_desc(native, cfg, module))
    assert st["n_tokens"] == lay.n_tokens
    assert st["n_windows"] == len(lay.windows)
    assert st["max_tokens"] == max(w.n for w in lay.windows)
    assert st["allowed_pairs"] == O.allowed_pairs(lay)
    assert st["n_masked"] == sum(len(np.unique(lay.labels[w.tok_off:w.tok_off + w.n])) > 1 for w in lay.windows)


def test_host_index_map_random_small_grids(native):
    rng = np.random.default_rng(3)
    for _ in range(40):
        nd = int(rng.integers(2, 4))
        grid = [1 if nd == 2 else int(rng.integers(1, 7))] + [int(rng.integers(1, 20)) for _ in range(2)]
        win = [int(rng.integers(1, g + 1)) for g in grid]
        if nd == 2:
            win[0] = 1
        sh = [int(rng.integers(0, w)) for w in win]
        if nd == 2:
            sh[0] = 0
        per = int(rng.integers(0, 8))
        b = int(rng.integers(1, 3))
        d = native.make_desc(b, grid, 8, 1, win, sh, per, native.SWIN_F32, ndim=nd)
        lay = O.window_layout(b, grid, win, sh, per)
        m, lab = native.swin_attn_host_index_map(d)
        assert np.array_equal(m, lay.perm), (grid, win, sh, per)
        assert np.array_equal(lab, lay.labels), (grid, win, sh, per)


def _status(native, **kw):
    base = dict(batch=1, grid=(1, 8, 8), channels=64, heads=2, window=(1, 4, 4), shift=(0, 2, 2),
                periodic=4, dtype=native.SWIN_BF16)
    base.update(kw)
    d = native.make_desc(**base)
    st = native.SwinAttnStats()
    return native.lib.swin_attn_host_stats(ctypes.byref(d), ctypes.byref(st))


def test_descriptor_errors(native):
    ARG = 1
    assert _status(native) == 0
    assert _status(native, shift=(0, 4, 2)) == ARG          # shift >= window
    assert _status(native, window=(1, 9, 4)) == ARG         # window > grid
    assert _status(native, channels=63) == ARG              # C % heads
    assert _status(native, batch=0) == ARG
    assert _status(native, periodic=8) == ARG
    assert _status(native, dtype=7) == ARG
    assert native.lib.swin_attn_host_stats(None, ctypes.byref(native.SwinAttnStats())) == ARG


def test_plan_create_rejects_before_touching_the_device(native):
    UNSUP = 2
    h = ctypes.c_void_p()
    d = native.make_desc(1, (1, 8, 8), 64, 4, (1, 4, 4), (0, 2, 2))   # head_dim 16 in bf16
    assert native.lib.swin_attn_plan_create(ctypes.byref(d), ctypes.byref(h)) == UNSUP
    assert h.value is None
    assert b"head_dim" in native.lib.swin_attn_last_error()
    d = native.make_desc(1, (1, 8, 8), 96, 1, (1, 4, 4), (0, 2, 2))   # head_dim 96 in bf16
    assert native.lib.swin_attn_plan_create(ctypes.byref(d), ctypes.byref(h)) == UNSUP
    d = native.make_desc(1, (1, 32, 32), 64, 2, (1, 17, 16), (0, 0, 0), dtype=native.SWIN_F32)  # 272 tokens, fp32
    assert native.lib.swin_attn_plan_create(ctypes.byref(d), ctypes.byref(h)) == UNSUP
    assert b"256" in native.lib.swin_attn_last_error()


def test_status_strings(native):
    for s in range(5):
        assert native.swin_status_string(s).startswith("SWIN_")


def test_binding_buffer_checks_without_gpu(native):
    """The binding refuses, before any library call, tensors that are not on a GPU, not
    tensors at all, or (checked on CPU tensors' size path through the same function) too small;
    None is passed through to the library's NULL checks."""
    import torch
    native.check_buffer(None, "x", 1 << 40)
    with pytest.raises(TypeError):
        native.check_buffer(np.zeros(4, dtype=np.float32), "x", 16)
    with pytest.raises(ValueError, match="GPU"):
        native.check_buffer(torch.zeros(4), "x", 16)
