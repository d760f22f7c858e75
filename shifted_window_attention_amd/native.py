"""ctypes declarations of the C ABI (include/swin_attn.h, include/swin_block.h,
include/swin_offload.h, include/swin_route.h) and argument marshalling.

Functions take torch tensors (device memory, already allocated by the caller)
and pass their data pointers and the current HIP stream to the library.
Host-only entry points (index map, stats) take numpy arrays.
"""
import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libswinattn.so")

SWIN_OK = 0
SWIN_F32 = 0
SWIN_BF16 = 1
SWIN_PERIODIC_LEVEL = 0x1
SWIN_PERIODIC_LAT = 0x2
SWIN_PERIODIC_LON = 0x4


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
    if not os.path.exists(LIB_PATH):
        raise ImportError("libswinattn.so is not built: run `python -c 'import __graft_entry__ as g; g.build()'` "
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
        "swin_attn_sizes": (st, [vp, P(sz), P(sz), P(sz)]),
        "swin_attn_fwd": (st, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "swin_attn_bwd": (st, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "swin_window_gather": (st, [vp, vp, vp, vp]),
        "swin_window_scatter": (st, [vp, vp, vp, vp]),
        "swin_attn_trace_events": (st, [P(vp), st]),
        "swin_attn_trace_cursor": (st, []),
        "swin_block_plan_create": (st, [P(SwinBlockDesc), P(vp)]),
        "swin_block_plan_destroy": (None, [vp]),
        "swin_block_sizes": (st, [vp, P(sz), P(sz), P(sz)]),
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
    return h


def swin_attn_plan_destroy(plan):
    lib.swin_attn_plan_destroy(plan)


def swin_attn_plan_stats(plan):
    st = SwinAttnStats()
    _check(lib.swin_attn_plan_stats(plan, ctypes.byref(st)), "swin_attn_plan_stats")
    return st.as_dict()


def swin_attn_sizes(plan):
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.swin_attn_sizes(plan, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)), "swin_attn_sizes")
    return a.value, b.value, c.value


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def swin_attn_fwd(plan, x, w_qkv, b_qkv, w_proj, b_proj, bias_table, y, saved, ws=None, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.swin_attn_fwd(plan, _ptr(x), _ptr(w_qkv), _ptr(b_qkv), _ptr(w_proj), _ptr(b_proj), _ptr(bias_table),
                             _ptr(y), _ptr(saved), _ptr(ws), ws_bytes, _stream(stream)), "swin_attn_fwd")


def swin_attn_bwd(plan, dy, x, w_qkv, w_proj, bias_table, saved, dx, dw_qkv, db_qkv, dw_proj, db_proj, dbias_table,
                  ws, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.swin_attn_bwd(plan, _ptr(dy), _ptr(x), _ptr(w_qkv), _ptr(w_proj), _ptr(bias_table), _ptr(saved),
                             _ptr(dx), _ptr(dw_qkv), _ptr(db_qkv), _ptr(dw_proj), _ptr(db_proj), _ptr(dbias_table),
                             _ptr(ws), ws_bytes, _stream(stream)), "swin_attn_bwd")


def swin_attn_trace_events(events):
    """events: a ctypes array of hipEvent_t handles (or None to uninstall)."""
    if events is None:
        _check(lib.swin_attn_trace_events(None, 0), "swin_attn_trace_events")
    else:
        _check(lib.swin_attn_trace_events(events, len(events)), "swin_attn_trace_events")


def swin_attn_trace_cursor():
    return int(lib.swin_attn_trace_cursor())


def swin_window_gather(plan, x, xw, stream=None):
    _check(lib.swin_window_gather(plan, _ptr(x), _ptr(xw), _stream(stream)), "swin_window_gather")


def swin_window_scatter(plan, yw, y, stream=None):
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
    return h


def swin_block_plan_destroy(plan):
    lib.swin_block_plan_destroy(plan)


def swin_block_sizes(plan):
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.swin_block_sizes(plan, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)), "swin_block_sizes")
    return a.value, b.value, c.value


def swin_block_fwd(plan, x, params, y, saved, ws=None, stream=None):
    """params: mapping from field name (ln1_g, ..., b2) to a device tensor or None."""
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    prm = _struct_of(SwinBlockParams, params)
    _check(lib.swin_block_fwd(plan, _ptr(x), ctypes.byref(prm), _ptr(y), _ptr(saved), _ptr(ws), ws_bytes,
                              _stream(stream)), "swin_block_fwd")


def swin_block_bwd(plan, dy, x, params, saved, dx, grads, ws, stream=None):
    """params as for swin_block_fwd; grads: the same names mapped to fp32 device tensors (None: NULL)."""
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


def swin_offload_store(engine, dev, host, nbytes, after=None):
    t = ctypes.c_uint64()
    _check(lib.swin_offload_store(engine, _addr(dev), _addr(host), nbytes, _stream(after), ctypes.byref(t)),
           "swin_offload_store")
    return t.value


def swin_offload_load(engine, host, dev, nbytes, after=None):
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
    _check(lib.swin_route_pack(plan.handle, int(p), _ptr(local), _ptr(send), _stream(stream)), "swin_route_pack")


def swin_route_unpack(plan, r, recv, local, stream=None):
    _check(lib.swin_route_unpack(plan.handle, int(r), _ptr(recv), _ptr(local), _stream(stream)), "swin_route_unpack")


def swin_route_loopback(plan, sends, recvs, stream=None):
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
