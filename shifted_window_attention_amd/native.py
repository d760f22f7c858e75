"""ctypes declarations of the C ABI (include/swin_attn.h, include/swin_block.h,
include/swin_offload.h, include/swin_route.h) and argument marshalling.

Functions take torch tensors (device memory, already allocated by the caller)
and pass their data pointers and the current HIP stream to the library.
Host-only entry points (index map, stats) take numpy arrays.

The C functions receive bare pointers and cannot see how large a buffer is, so
before a device call this layer checks every tensor it passes against the
plan's shapes: on a GPU, contiguous, of the element type the header names and
at least as many bytes as the call reads or writes (a ValueError or TypeError
otherwise, and nothing is launched). NULL pointers, aliasing, workspace sizes
and rank numbers are left to the library's own checks, which report them as a
status (SwinError).
"""
import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# SWIN_ATTN_LIB names another build of the same library (the host-only sanitizer build of the
# host tests); unset, the in-tree libswinattn.so is loaded.
LIB_PATH = os.environ.get("SWIN_ATTN_LIB") or os.path.join(_PKG, "libswinattn.so")

SWIN_OK = 0
SWIN_F32 = 0
SWIN_BF16 = 1
SWIN_PERIODIC_LEVEL = 0x1
SWIN_PERIODIC_LAT = 0x2
SWIN_PERIODIC_LON = 0x4
SWIN_FLAG_DT_SATURATED = 0x1


class SwinError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = "%s: %s (%s)" % (where, lib.swin_status_string(status).decode(), lib.swin_attn_last_error().decode())
        super().__init__(msg)


class SwinAttnDesc(ctypes.Structure):
    _fields_ = [("ndim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("batch", ctypes.c_int64),
                ("grid", ctypes.c_int64 * 3), ("channels", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("window", ctypes.c_int32 * 3), ("shift", ctypes.c_int32 * 3), ("periodic", ctypes.c_uint32),
                ("scale", ctypes.c_float)]


class SwinAttnStats(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("n_windows", ctypes.c_int64), ("n_masked", ctypes.c_int64),
                ("n_classes", ctypes.c_int64), ("max_tokens", ctypes.c_int64), ("allowed_pairs", ctypes.c_int64)]

    def as_dict(self):
        return {f: int(getattr(self, f)) for f, _ in self._fields_}


class SwinBlockDesc(ctypes.Structure):
    _fields_ = [("attn", SwinAttnDesc), ("hidden", ctypes.c_int32), ("ln_eps", ctypes.c_float)]


_BLOCK_PARAM_FIELDS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_proj", "b_proj", "bias_table", "ln2_g", "ln2_b", "w1",
                       "b1", "w2", "b2")


class SwinBlockParams(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in _BLOCK_PARAM_FIELDS]


class SwinBlockGrads(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in _BLOCK_PARAM_FIELDS]


SWIN_LAYOUT_STRIPES = 0
SWIN_LAYOUT_WINDOWS = 1


class SwinRankLayout(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("ranks", ctypes.c_int32), ("shift", ctypes.c_int32 * 3)]


def make_rank_layout(kind, ranks, shift=(0, 0, 0)):
    lay = SwinRankLayout()
    lay.kind = int(kind)
    lay.ranks = int(ranks)
    shift = tuple(int(v) for v in shift)
    if len(shift) == 2:
        shift = (0,) + shift
    for a in range(3):
        lay.shift[a] = shift[a]
    return lay


def _load():
    # One HIP runtime per process: torch ships its own. Importing it before the library makes
    # the library bind to that runtime; loaded first, the library would pull in the system
    # runtime, and torch's copy, loaded later, then finds no device.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(LIB_PATH + " is not built: run `python -c 'import __graft_entry__ as g; g.build()'` "
                          "or `python shifted_window_attention_amd/build_lib.py`")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    P = ctypes.POINTER
    sigs = {
        "swin_attn_host_index_map": (st, [P(SwinAttnDesc), P(ctypes.c_int64), P(ctypes.c_uint8)]),
        "swin_attn_host_stats": (st, [P(SwinAttnDesc), P(SwinAttnStats)]),
        "swin_attn_plan_create": (st, [P(SwinAttnDesc), P(vp)]),
        "swin_attn_plan_destroy": (None, [vp]),
        "swin_attn_plan_stats": (st, [vp, P(SwinAttnStats)]),
        "swin_attn_index_map": (st, [vp, P(ctypes.c_int64), P(ctypes.c_uint8)]),
        "swin_attn_sizes": (st, [vp, P(sz), P(sz), P(sz)]),
        "swin_attn_plan_flags": (st, [vp, P(ctypes.c_uint32), st]),
        "swin_attn_fwd": (st, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "swin_attn_bwd": (st, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "swin_attn_bwd_noalloc": (st, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "swin_attn_sizes_recompute": (st, [vp, P(sz), P(sz), P(sz)]),
        "swin_attn_fwd_recompute": (st, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "swin_attn_bwd_recompute": (st, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "swin_window_gather": (st, [vp, vp, vp, vp]),
        "swin_window_scatter": (st, [vp, vp, vp, vp]),
        "swin_attn_trace_events": (st, [P(vp), st]),
        "swin_attn_trace_cursor": (st, []),
        "swin_block_plan_create": (st, [P(SwinBlockDesc), P(vp)]),
        "swin_block_plan_destroy": (None, [vp]),
        "swin_block_sizes": (st, [vp, P(sz), P(sz), P(sz)]),
        "swin_block_plan_flags": (st, [vp, P(ctypes.c_uint32), st]),
        "swin_block_fwd": (st, [vp, vp, P(SwinBlockParams), vp, vp, vp, sz, vp]),
        "swin_block_bwd": (st, [vp, vp, vp, P(SwinBlockParams), vp, vp, P(SwinBlockGrads), vp, sz, vp]),
        "swin_offload_create": (st, [ctypes.c_int32, P(vp)]),
        "swin_offload_destroy": (None, [vp]),
        "swin_pinned_alloc": (st, [sz, P(vp)]),
        "swin_pinned_free": (st, [vp]),
        "swin_offload_store": (st, [vp, vp, vp, sz, vp, P(ctypes.c_uint64)]),
        "swin_offload_load": (st, [vp, vp, vp, sz, vp, P(ctypes.c_uint64)]),
        "swin_offload_wait": (st, [vp, ctypes.c_uint64, vp]),
        "swin_offload_query": (st, [vp, ctypes.c_uint64, P(ctypes.c_int32)]),
        "swin_offload_sync": (st, [vp]),
        "swin_offload_bytes": (st, [vp, P(ctypes.c_uint64), P(ctypes.c_uint64)]),
        "swin_route_plan_create": (st, [P(SwinAttnDesc), P(SwinRankLayout), P(SwinRankLayout), P(vp)]),
        "swin_route_plan_destroy": (None, [vp]),
        "swin_route_counts": (st, [vp, P(ctypes.c_int64), P(ctypes.c_int64), P(ctypes.c_int64)]),
        "swin_route_host_tables": (st, [P(SwinAttnDesc), P(SwinRankLayout), P(SwinRankLayout), P(ctypes.c_int64),
                                        P(ctypes.c_int32), P(ctypes.c_int32)]),
        "swin_route_pack": (st, [vp, ctypes.c_int32, vp, vp, vp]),
        "swin_route_unpack": (st, [vp, ctypes.c_int32, vp, vp, vp]),
        "swin_route_loopback": (st, [vp, P(vp), P(vp), vp]),
        "swin_status_string": (ctypes.c_char_p, [st]),
        "swin_attn_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


lib = _load()


def _check(status, where):
    if status != SWIN_OK:
        raise SwinError(status, where)


_ELEM_BYTES = {SWIN_F32: 4, SWIN_BF16: 2}


def _torch_dtype(code):
    import torch
    return {SWIN_F32: torch.float32, SWIN_BF16: torch.bfloat16}.get(code)


def check_buffer(t, what, nbytes, dtype=None):
    """Checks that tensor t (None is passed through to the library's NULL checks) is a contiguous
    GPU tensor of at least nbytes bytes and, when dtype is given, of that element type."""
    if t is None:
        return
    if not (hasattr(t, "data_ptr") and hasattr(t, "is_cuda")):
        raise TypeError("%s: expected a torch tensor, got %s" % (what, type(t).__name__))
    if not t.is_cuda:
        raise ValueError("%s: must be a GPU tensor (device %s)" % (what, t.device))
    if not t.is_contiguous():
        raise ValueError("%s: must be contiguous" % what)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s: expected %s, got %s" % (what, dtype, t.dtype))
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError("%s: %d bytes, the call needs %d" % (what, have, nbytes))


class _AttnShape:
    """What the buffer checks need to know of an attention plan."""

    def __init__(self, desc, n_tokens, saved_bytes):
        self.n_tok = int(n_tokens)
        self.C = int(desc.channels)
        w = [int(desc.window[a]) for a in range(3)]
        self.table = int(desc.heads) * (2 * w[0] - 1) * (2 * w[1] - 1) * (2 * w[2] - 1)
        self.dtype_code = int(desc.dtype)
        self.elem = _ELEM_BYTES.get(self.dtype_code, 2)
        self.saved_bytes = int(saved_bytes)


_ATTN_SHAPES = {}   # plan handle value -> _AttnShape
_BLOCK_SHAPES = {}  # block plan handle value -> (_AttnShape, hidden)


def _key(handle):
    if handle is None:
        return None
    return handle.value if isinstance(handle, ctypes.c_void_p) else int(handle)


def make_desc(batch, grid, channels, heads, window, shift, periodic=SWIN_PERIODIC_LON, dtype=SWIN_BF16,
              scale=0.0, ndim=None):
    d = SwinAttnDesc()
    grid = tuple(int(g) for g in grid)
    window = tuple(int(w) for w in window)
    shift = tuple(int(s) for s in shift)
    if len(grid) == 2:
        grid, window, shift = (1,) + grid, (1,) + window, (0,) + shift
    d.ndim = int(ndim) if ndim is not None else (2 if grid[0] == 1 and window[0] == 1 and shift[0] == 0 else 3)
    d.dtype = int(dtype)
    d.batch = int(batch)
    for a in range(3):
        d.grid[a] = grid[a]
        d.window[a] = window[a]
        d.shift[a] = shift[a]
    d.channels = int(channels)
    d.heads = int(heads)
    d.periodic = int(periodic)
    d.scale = float(scale)
    return d


def swin_attn_host_index_map(desc):
    st = SwinAttnStats()
    _check(lib.swin_attn_host_stats(ctypes.byref(desc), ctypes.byref(st)), "swin_attn_host_stats")
    n = st.n_tokens
    m = np.empty(n, dtype=np.int64)
    lab = np.empty(n, dtype=np.uint8)
    _check(lib.swin_attn_host_index_map(ctypes.byref(desc), m.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                        lab.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))),
           "swin_attn_host_index_map")
    return m, lab


def swin_attn_host_stats(desc):
    st = SwinAttnStats()
    _check(lib.swin_attn_host_stats(ctypes.byref(desc), ctypes.byref(st)), "swin_attn_host_stats")
    return st.as_dict()


def swin_status_string(status):
    return lib.swin_status_string(status).decode()


def swin_attn_plan_create(desc):
    h = ctypes.c_void_p()
    _check(lib.swin_attn_plan_create(ctypes.byref(desc), ctypes.byref(h)), "swin_attn_plan_create")
    _, _, saved = swin_attn_sizes(h)
    _ATTN_SHAPES[h.value] = _AttnShape(desc, swin_attn_plan_stats(h)["n_tokens"], saved)
    return h


def swin_attn_plan_destroy(plan):
    _ATTN_SHAPES.pop(_key(plan), None)
    lib.swin_attn_plan_destroy(plan)


def swin_attn_plan_stats(plan):
    st = SwinAttnStats()
    _check(lib.swin_attn_plan_stats(plan, ctypes.byref(st)), "swin_attn_plan_stats")
    return st.as_dict()


def swin_attn_index_map(plan):
    """The plan's slot -> grid map and wrap labels (host copies, no device call)."""
    n = swin_attn_plan_stats(plan)["n_tokens"]
    m = np.empty(n, dtype=np.int64)
    lab = np.empty(n, dtype=np.uint8)
    _check(lib.swin_attn_index_map(plan, m.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                   lab.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))), "swin_attn_index_map")
    return m, lab


def swin_attn_sizes(plan):
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.swin_attn_sizes(plan, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)), "swin_attn_sizes")
    return a.value, b.value, c.value


def swin_attn_plan_flags(plan, clear=False):
    """Sticky SWIN_FLAG_* bits of the plan (waits for the device); clear=True resets them."""
    f = ctypes.c_uint32()
    _check(lib.swin_attn_plan_flags(plan, ctypes.byref(f), 1 if clear else 0), "swin_attn_plan_flags")
    return f.value


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check_attn_weights(sh, w_qkv, b_qkv, w_proj, b_proj, bias_table):
    dt, e, C = _torch_dtype(sh.dtype_code), sh.elem, sh.C
    check_buffer(w_qkv, "w_qkv", 3 * C * C * e, dt)
    check_buffer(b_qkv, "b_qkv", 3 * C * e, dt)
    check_buffer(w_proj, "w_proj", C * C * e, dt)
    check_buffer(b_proj, "b_proj", C * e, dt)
    check_buffer(bias_table, "bias_table", sh.table * 4, _torch_dtype(SWIN_F32))


def swin_attn_fwd(plan, x, w_qkv, b_qkv, w_proj, b_proj, bias_table, y, saved, ws=None, stream=None):
    sh = _ATTN_SHAPES.get(_key(plan))
    if sh is not None:
        rows = sh.n_tok * sh.C * sh.elem
        check_buffer(x, "x", rows, _torch_dtype(sh.dtype_code))
        check_buffer(y, "y", rows, _torch_dtype(sh.dtype_code))
        _check_attn_weights(sh, w_qkv, b_qkv, w_proj, b_proj, bias_table)
        check_buffer(saved, "saved", sh.saved_bytes)
        check_buffer(ws, "ws", 0)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.swin_attn_fwd(plan, _ptr(x), _ptr(w_qkv), _ptr(b_qkv), _ptr(w_proj), _ptr(b_proj), _ptr(bias_table),
                             _ptr(y), _ptr(saved), _ptr(ws), ws_bytes, _stream(stream)), "swin_attn_fwd")


def swin_attn_bwd(plan, dy, x, w_qkv, w_proj, bias_table, saved, dx, dw_qkv, db_qkv, dw_proj, db_proj, dbias_table,
                  ws, stream=None):
    sh = _ATTN_SHAPES.get(_key(plan))
    if sh is not None:
        rows, dt, f32, C = sh.n_tok * sh.C * sh.elem, _torch_dtype(sh.dtype_code), _torch_dtype(SWIN_F32), sh.C
        for t, what in ((dy, "dy"), (x, "x"), (dx, "dx")):
            check_buffer(t, what, rows, dt)
        _check_attn_weights(sh, w_qkv, None, w_proj, None, bias_table)
        check_buffer(saved, "saved", sh.saved_bytes)
        check_buffer(dw_qkv, "dw_qkv", 3 * C * C * 4, f32)
        check_buffer(db_qkv, "db_qkv", 3 * C * 4, f32)
        check_buffer(dw_proj, "dw_proj", C * C * 4, f32)
        check_buffer(db_proj, "db_proj", C * 4, f32)
        check_buffer(dbias_table, "dbias_table", sh.table * 4, f32)
        check_buffer(ws, "ws", 0)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.swin_attn_bwd(plan, _ptr(dy), _ptr(x), _ptr(w_qkv), _ptr(w_proj), _ptr(bias_table), _ptr(saved),
                             _ptr(dx), _ptr(dw_qkv), _ptr(db_qkv), _ptr(dw_proj), _ptr(db_proj), _ptr(dbias_table),
                             _ptr(ws), ws_bytes, _stream(stream)), "swin_attn_bwd")


def swin_attn_sizes_recompute(plan):
    """(fwd_ws, bwd_ws, saved_bytes) of the recomputing forward/backward pair."""
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.swin_attn_sizes_recompute(plan, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)),
           "swin_attn_sizes_recompute")
    return a.value, b.value, c.value


def swin_attn_fwd_recompute(plan, x, w_qkv, b_qkv, w_proj, b_proj, bias_table, y, saved, ws, stream=None):
    """swin_attn_fwd keeping only [o | LSE] in saved; ws (fwd_ws bytes) takes the q/k/v planes."""
    sh = _ATTN_SHAPES.get(_key(plan))
    if sh is not None:
        _, _, saved_bytes = swin_attn_sizes_recompute(plan)
        rows = sh.n_tok * sh.C * sh.elem
        check_buffer(x, "x", rows, _torch_dtype(sh.dtype_code))
        check_buffer(y, "y", rows, _torch_dtype(sh.dtype_code))
        _check_attn_weights(sh, w_qkv, b_qkv, w_proj, b_proj, bias_table)
        check_buffer(saved, "saved", saved_bytes)
        check_buffer(ws, "ws", 0)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.swin_attn_fwd_recompute(plan, _ptr(x), _ptr(w_qkv), _ptr(b_qkv), _ptr(w_proj), _ptr(b_proj),
                                       _ptr(bias_table), _ptr(y), _ptr(saved), _ptr(ws), ws_bytes, _stream(stream)),
           "swin_attn_fwd_recompute")


def swin_attn_bwd_recompute(plan, dy, x, w_qkv, b_qkv, w_proj, bias_table, saved, dx, dw_qkv, db_qkv, dw_proj,
                            db_proj, dbias_table, ws, stream=None):
    """swin_attn_bwd that rebuilds q/k/v from x (and b_qkv) into ws before the backward."""
    sh = _ATTN_SHAPES.get(_key(plan))
    if sh is not None:
        _, _, saved_bytes = swin_attn_sizes_recompute(plan)
        rows, dt, f32, C = sh.n_tok * sh.C * sh.elem, _torch_dtype(sh.dtype_code), _torch_dtype(SWIN_F32), sh.C
        for t, what in ((dy, "dy"), (x, "x"), (dx, "dx")):
            check_buffer(t, what, rows, dt)
        _check_attn_weights(sh, w_qkv, b_qkv, w_proj, None, bias_table)
        check_buffer(saved, "saved", saved_bytes)
        check_buffer(dw_qkv, "dw_qkv", 3 * C * C * 4, f32)
        check_buffer(db_qkv, "db_qkv", 3 * C * 4, f32)
        check_buffer(dw_proj, "dw_proj", C * C * 4, f32)
        check_buffer(db_proj, "db_proj", C * 4, f32)
        check_buffer(dbias_table, "dbias_table", sh.table * 4, f32)
        check_buffer(ws, "ws", 0)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.swin_attn_bwd_recompute(plan, _ptr(dy), _ptr(x), _ptr(w_qkv), _ptr(b_qkv), _ptr(w_proj),
                                       _ptr(bias_table), _ptr(saved), _ptr(dx), _ptr(dw_qkv), _ptr(db_qkv),
                                       _ptr(dw_proj), _ptr(db_proj), _ptr(dbias_table), _ptr(ws), ws_bytes,
                                       _stream(stream)), "swin_attn_bwd_recompute")


SWIN_NOALLOC_SCRATCH_BYTES = 64 << 20


def swin_attn_bwd_noalloc(plan, dy, x, w_qkv, w_proj, bias_table, saved, dx, dw_qkv, db_qkv, dw_proj, db_proj,
                          dbias_table, stream=None):
    """swin_attn_bwd on the library's own per-GPU scratch array (no workspace argument)."""
    sh = _ATTN_SHAPES.get(_key(plan))
    if sh is not None:
        rows, dt, f32, C = sh.n_tok * sh.C * sh.elem, _torch_dtype(sh.dtype_code), _torch_dtype(SWIN_F32), sh.C
        for t, what in ((dy, "dy"), (x, "x"), (dx, "dx")):
            check_buffer(t, what, rows, dt)
        _check_attn_weights(sh, w_qkv, None, w_proj, None, bias_table)
        check_buffer(saved, "saved", sh.saved_bytes)
        check_buffer(dw_qkv, "dw_qkv", 3 * C * C * 4, f32)
        check_buffer(db_qkv, "db_qkv", 3 * C * 4, f32)
        check_buffer(dw_proj, "dw_proj", C * C * 4, f32)
        check_buffer(db_proj, "db_proj", C * 4, f32)
        check_buffer(dbias_table, "dbias_table", sh.table * 4, f32)
    _check(lib.swin_attn_bwd_noalloc(plan, _ptr(dy), _ptr(x), _ptr(w_qkv), _ptr(w_proj), _ptr(bias_table),
                                     _ptr(saved), _ptr(dx), _ptr(dw_qkv), _ptr(db_qkv), _ptr(dw_proj), _ptr(db_proj),
                                     _ptr(dbias_table), _stream(stream)), "swin_attn_bwd_noalloc")


def swin_attn_trace_events(events):
    """events: a ctypes array of hipEvent_t handles (or None to uninstall)."""
    if events is None:
        _check(lib.swin_attn_trace_events(None, 0), "swin_attn_trace_events")
    else:
        _check(lib.swin_attn_trace_events(events, len(events)), "swin_attn_trace_events")


def swin_attn_trace_cursor():
    return int(lib.swin_attn_trace_cursor())


def _check_rows(plan, pairs):
    # gather/scatter move rows bit for bit: any element type of the row's byte size will do
    sh = _ATTN_SHAPES.get(_key(plan))
    if sh is not None:
        for t, what in pairs:
            check_buffer(t, what, sh.n_tok * sh.C * sh.elem)


def swin_window_gather(plan, x, xw, stream=None):
    _check_rows(plan, ((x, "x"), (xw, "xw")))
    _check(lib.swin_window_gather(plan, _ptr(x), _ptr(xw), _stream(stream)), "swin_window_gather")


def swin_window_scatter(plan, yw, y, stream=None):
    _check_rows(plan, ((yw, "yw"), (y, "y")))
    _check(lib.swin_window_scatter(plan, _ptr(yw), _ptr(y), _stream(stream)), "swin_window_scatter")


def make_block_desc(attn_desc, hidden=0, ln_eps=0.0):
    d = SwinBlockDesc()
    d.attn = attn_desc
    d.hidden = int(hidden)
    d.ln_eps = float(ln_eps)
    return d


def _struct_of(cls, tensors):
    """tensors: a mapping from field name to a tensor or None (NULL)."""
    unknown = set(tensors) - set(_BLOCK_PARAM_FIELDS)
    if unknown:
        raise KeyError("unknown block fields: %s" % sorted(unknown))
    s = cls()
    for f in _BLOCK_PARAM_FIELDS:
        t = tensors.get(f)
        setattr(s, f, None if t is None else t.data_ptr())
    return s


def swin_block_plan_create(desc):
    h = ctypes.c_void_p()
    _check(lib.swin_block_plan_create(ctypes.byref(desc), ctypes.byref(h)), "swin_block_plan_create")
    _, _, saved = swin_block_sizes(h)
    n_tok = swin_attn_host_stats(desc.attn)["n_tokens"]
    hidden = int(desc.hidden) if desc.hidden > 0 else 4 * int(desc.attn.channels)
    _BLOCK_SHAPES[h.value] = (_AttnShape(desc.attn, n_tok, saved), hidden)
    return h


def swin_block_plan_destroy(plan):
    _BLOCK_SHAPES.pop(_key(plan), None)
    lib.swin_block_plan_destroy(plan)


def _block_param_bytes(C, hidden, table):
    """Elements of every block parameter (the same for its fp32 gradient)."""
    return {"ln1_g": C, "ln1_b": C, "w_qkv": 3 * C * C, "b_qkv": 3 * C, "w_proj": C * C, "b_proj": C,
            "bias_table": table, "ln2_g": C, "ln2_b": C, "w1": hidden * C, "b1": hidden, "w2": C * hidden, "b2": C}


def _check_block(plan, acts, params, grads=None, saved=None, ws=None):
    entry = _BLOCK_SHAPES.get(_key(plan))
    if entry is None:
        return
    sh, hidden = entry
    bf16, f32 = _torch_dtype(SWIN_BF16), _torch_dtype(SWIN_F32)
    for t, what in acts:
        check_buffer(t, what, sh.n_tok * sh.C * 2, bf16)
    n = _block_param_bytes(sh.C, hidden, sh.table)
    for f, t in params.items():
        if f in n:
            check_buffer(t, f, n[f] * (4 if f == "bias_table" else 2), f32 if f == "bias_table" else bf16)
    for f, t in (grads or {}).items():
        if f in n:
            check_buffer(t, "grad " + f, n[f] * 4, f32)
    check_buffer(saved, "saved", sh.saved_bytes)
    check_buffer(ws, "ws", 0)


def swin_block_sizes(plan):
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.swin_block_sizes(plan, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)), "swin_block_sizes")
    return a.value, b.value, c.value


def swin_block_plan_flags(plan, clear=False):
    """Sticky SWIN_FLAG_* bits of the block's attention module (waits for the device)."""
    f = ctypes.c_uint32()
    _check(lib.swin_block_plan_flags(plan, ctypes.byref(f), 1 if clear else 0), "swin_block_plan_flags")
    return f.value


def swin_block_fwd(plan, x, params, y, saved, ws=None, stream=None):
    """params: mapping from field name (ln1_g, ..., b2) to a device tensor or None."""
    _check_block(plan, ((x, "x"), (y, "y")), params, saved=saved, ws=ws)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    prm = _struct_of(SwinBlockParams, params)
    _check(lib.swin_block_fwd(plan, _ptr(x), ctypes.byref(prm), _ptr(y), _ptr(saved), _ptr(ws), ws_bytes,
                              _stream(stream)), "swin_block_fwd")


def swin_block_bwd(plan, dy, x, params, saved, dx, grads, ws, stream=None):
    """params as for swin_block_fwd; grads: the same names mapped to fp32 device tensors (None: NULL)."""
    _check_block(plan, ((dy, "dy"), (x, "x"), (dx, "dx")), params, grads, saved=saved, ws=ws)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    prm = _struct_of(SwinBlockParams, params)
    grd = _struct_of(SwinBlockGrads, grads)
    _check(lib.swin_block_bwd(plan, _ptr(dy), _ptr(x), ctypes.byref(prm), _ptr(saved), _ptr(dx), ctypes.byref(grd),
                              _ptr(ws), ws_bytes, _stream(stream)), "swin_block_bwd")


class BlockPlan:
    """Owns a block plan handle; allocates its saved state and backward workspace with torch on request."""

    def __init__(self, desc, device="cuda"):
        import torch
        self.desc = desc
        self.handle = swin_block_plan_create(desc)
        self.fwd_ws, self.bwd_ws, self.saved_bytes = swin_block_sizes(self.handle)
        self.device = device
        self._torch = torch

    def alloc_saved(self):
        return self._torch.empty(max(self.saved_bytes, 1), dtype=self._torch.uint8, device=self.device)

    def alloc_bwd_ws(self):
        return self._torch.empty(max(self.bwd_ws, 1), dtype=self._torch.uint8, device=self.device)

    def close(self):
        if self.handle is not None:
            swin_block_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _addr(p):
    """A device tensor, a pinned-host buffer (PinnedBuffer) or a raw address -> c_void_p."""
    if p is None:
        return None
    if hasattr(p, "data_ptr"):
        return ctypes.c_void_p(p.data_ptr())
    if isinstance(p, PinnedBuffer):
        return ctypes.c_void_p(p.ptr)
    return ctypes.c_void_p(int(p))


class PinnedBuffer:
    """Pinned host memory from swin_pinned_alloc; .array is a uint8 numpy view of it."""

    def __init__(self, nbytes):
        h = ctypes.c_void_p()
        _check(lib.swin_pinned_alloc(nbytes, ctypes.byref(h)), "swin_pinned_alloc")
        self.ptr = h.value
        self.nbytes = nbytes
        self.array = np.ctypeslib.as_array((ctypes.c_uint8 * nbytes).from_address(self.ptr))

    def free(self):
        if self.ptr:
            self.array = None
            _check(lib.swin_pinned_free(ctypes.c_void_p(self.ptr)), "swin_pinned_free")
            self.ptr = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def swin_offload_create(ring=0):
    h = ctypes.c_void_p()
    _check(lib.swin_offload_create(int(ring), ctypes.byref(h)), "swin_offload_create")
    return h


def swin_offload_destroy(engine):
    lib.swin_offload_destroy(engine)


def _check_span(p, what, nbytes):
    """Byte-size check of a device tensor or pinned buffer; raw addresses are passed through."""
    if isinstance(p, PinnedBuffer):
        if p.ptr and p.nbytes < nbytes:
            raise ValueError("%s: %d bytes, the call needs %d" % (what, p.nbytes, nbytes))
    elif p is not None and hasattr(p, "data_ptr"):
        check_buffer(p, what, nbytes)


def swin_offload_store(engine, dev, host, nbytes, after=None):
    _check_span(dev, "dev", nbytes)
    _check_span(host, "host", nbytes)
    t = ctypes.c_uint64()
    _check(lib.swin_offload_store(engine, _addr(dev), _addr(host), nbytes, _stream(after), ctypes.byref(t)),
           "swin_offload_store")
    return t.value


def swin_offload_load(engine, host, dev, nbytes, after=None):
    _check_span(host, "host", nbytes)
    _check_span(dev, "dev", nbytes)
    t = ctypes.c_uint64()
    _check(lib.swin_offload_load(engine, _addr(host), _addr(dev), nbytes, _stream(after), ctypes.byref(t)),
           "swin_offload_load")
    return t.value


def swin_offload_wait(engine, ticket, stream=None):
    _check(lib.swin_offload_wait(engine, ticket, _stream(stream)), "swin_offload_wait")


def swin_offload_query(engine, ticket):
    d = ctypes.c_int32()
    _check(lib.swin_offload_query(engine, ticket, ctypes.byref(d)), "swin_offload_query")
    return bool(d.value)


def swin_offload_sync(engine):
    _check(lib.swin_offload_sync(engine), "swin_offload_sync")


def swin_offload_bytes(engine):
    a, b = ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib.swin_offload_bytes(engine, ctypes.byref(a), ctypes.byref(b)), "swin_offload_bytes")
    return a.value, b.value


def _i64p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _i32p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def swin_route_host_tables(grid_desc, src, dst):
    """(counts [P, R], send_src [N_tok], recv_dst [N_tok]) of a route, computed on the host."""
    st = SwinAttnStats()
    d = SwinAttnDesc.from_buffer_copy(grid_desc)
    d.shift[0] = d.shift[1] = d.shift[2] = 0
    _check(lib.swin_attn_host_stats(ctypes.byref(d), ctypes.byref(st)), "swin_attn_host_stats")
    n = st.n_tokens
    counts = np.empty((src.ranks, dst.ranks), dtype=np.int64)
    send = np.empty(n, dtype=np.int32)
    recv = np.empty(n, dtype=np.int32)
    _check(lib.swin_route_host_tables(ctypes.byref(grid_desc), ctypes.byref(src), ctypes.byref(dst), _i64p(counts),
                                      _i32p(send), _i32p(recv)), "swin_route_host_tables")
    return counts, send, recv


class RoutePlan:
    """Owns a route plan handle and its sizes."""

    def __init__(self, grid_desc, src, dst):
        h = ctypes.c_void_p()
        _check(lib.swin_route_plan_create(ctypes.byref(grid_desc), ctypes.byref(src), ctypes.byref(dst),
                                          ctypes.byref(h)), "swin_route_plan_create")
        self.handle = h
        self.P, self.R = src.ranks, dst.ranks
        self.row_bytes = int(grid_desc.channels) * _ELEM_BYTES.get(int(grid_desc.dtype), 2)
        self.counts = np.empty((self.P, self.R), dtype=np.int64)
        self.src_sizes = np.empty(self.P, dtype=np.int64)
        self.dst_sizes = np.empty(self.R, dtype=np.int64)
        _check(lib.swin_route_counts(h, _i64p(self.counts), _i64p(self.src_sizes), _i64p(self.dst_sizes)),
               "swin_route_counts")

    def close(self):
        if self.handle is not None:
            lib.swin_route_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def swin_route_pack(plan, p, local, send, stream=None):
    if 0 <= int(p) < plan.P:  # other ranks: the library reports the error
        need = int(plan.src_sizes[int(p)]) * plan.row_bytes
        check_buffer(local, "local", need)
        check_buffer(send, "send", need)
    _check(lib.swin_route_pack(plan.handle, int(p), _ptr(local), _ptr(send), _stream(stream)), "swin_route_pack")


def swin_route_unpack(plan, r, recv, local, stream=None):
    if 0 <= int(r) < plan.R:
        need = int(plan.dst_sizes[int(r)]) * plan.row_bytes
        check_buffer(recv, "recv", need)
        check_buffer(local, "local", need)
    _check(lib.swin_route_unpack(plan.handle, int(r), _ptr(recv), _ptr(local), _stream(stream)), "swin_route_unpack")


def swin_route_loopback(plan, sends, recvs, stream=None):
    if len(sends) != plan.P or len(recvs) != plan.R:
        raise ValueError("swin_route_loopback: %d send and %d receive buffers for %d sources and %d destinations"
                         % (len(sends), len(recvs), plan.P, plan.R))
    for p, t in enumerate(sends):
        check_buffer(t, "send[%d]" % p, int(plan.src_sizes[p]) * plan.row_bytes)
    for r, t in enumerate(recvs):
        check_buffer(t, "recv[%d]" % r, int(plan.dst_sizes[r]) * plan.row_bytes)
    s_arr = (ctypes.c_void_p * len(sends))(*[None if t is None else t.data_ptr() for t in sends])
    r_arr = (ctypes.c_void_p * len(recvs))(*[None if t is None else t.data_ptr() for t in recvs])
    _check(lib.swin_route_loopback(plan.handle, s_arr, r_arr, _stream(stream)), "swin_route_loopback")


class Plan:
    """Owns a plan handle plus the device buffers it needs (saved state, backward workspace).

    Buffers are allocated here with torch (device memory plumbing); the library itself never allocates
    on the forward/backward path."""

    def __init__(self, desc, device="cuda"):
        import torch
        self.desc = desc
        self.handle = swin_attn_plan_create(desc)
        self.stats = swin_attn_plan_stats(self.handle)
        self.fwd_ws, self.bwd_ws, self.saved_bytes = swin_attn_sizes(self.handle)
        self.device = device
        self._torch = torch

    def alloc_saved(self):
        return self._torch.empty(max(self.saved_bytes, 1), dtype=self._torch.uint8, device=self.device)

    def alloc_bwd_ws(self):
        return self._torch.empty(max(self.bwd_ws, 1), dtype=self._torch.uint8, device=self.device)

    def close(self):
        if self.handle is not None:
            swin_attn_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
