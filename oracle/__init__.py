"""ctypes front-end of the plain C oracle (moe_oracle.h).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.  Arrays are numpy
arrays; every function mirrors one C entry point.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if _build.stale():
            _build.build()
        _lib = C.CDLL(_build.LIB)
        _declare(_lib)
    return _lib


def _p(a, ct):
    return a.ctypes.data_as(C.POINTER(ct))


class ExpertW(C.Structure):
    _fields_ = [("q_gate", C.c_void_p), ("s_gate", C.c_void_p),
                ("q_up", C.c_void_p), ("s_up", C.c_void_p),
                ("q_down", C.c_void_p), ("s_down", C.c_void_p)]


class MxExpertW(C.Structure):
    _fields_ = [("c_gate", C.c_void_p), ("e_gate", C.c_void_p),
                ("c_up", C.c_void_p), ("e_up", C.c_void_p),
                ("c_down", C.c_void_p), ("e_down", C.c_void_p)]


class CacheEvent(C.Structure):
    _fields_ = [("kind", C.c_int32), ("layer", C.c_int32),
                ("expert", C.c_int32), ("slot", C.c_int32)]


class CacheStats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in (
        "demand_hits", "demand_misses", "prefetch_issued", "prefetch_used",
        "prefetch_wasted", "prefetch_skipped", "prefetch_resident", "evictions",
        "pinned", "pin_fills")]


EV_HIT, EV_MISS, EV_PF_ISSUE, EV_PF_HIT, EV_PF_SKIP, EV_EVICT, EV_PIN_FILL, EV_PIN_KEEP = range(8)


def _declare(L):
    vp, i32, f32 = C.c_void_p, C.c_int, C.c_float
    L.orc_bf16_to_f32.argtypes = [C.c_uint16]
    L.orc_bf16_to_f32.restype = f32
    L.orc_f16_to_f32.argtypes = [C.c_uint16]
    L.orc_f16_to_f32.restype = f32
    L.orc_f32_to_bf16.argtypes = [f32]
    L.orc_f32_to_bf16.restype = C.c_uint16
    L.orc_e2m1_value.argtypes = [C.c_uint8]
    L.orc_e2m1_value.restype = f32
    L.orc_e8m0_value.argtypes = [C.c_uint8]
    L.orc_e8m0_value.restype = C.c_double
    L.orc_quant_row.argtypes = [vp, i32, vp, vp]
    L.orc_router.argtypes = [i32, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp, vp, vp]
    L.orc_proj_i4i8.argtypes = [vp, f32, vp, vp, i32, i32, i32, vp, i32, vp]
    L.orc_group_dots.argtypes = [vp, vp, i32, i32, i32, vp]
    L.orc_rows_exact_fp64.argtypes = [vp, i32, i32, i32]
    L.orc_rows_exact_fp64.restype = i32
    L.orc_expert.argtypes = [i32, i32, i32, vp, f32, C.POINTER(ExpertW), vp, i32, vp, vp, vp, vp]
    L.orc_layer.argtypes = [i32, i32, i32, i32, i32, i32, f32, vp, vp, vp,
                            C.POINTER(ExpertW), C.POINTER(ExpertW), vp, i32, vp, vp, vp]
    L.orc_proj_mx.argtypes = [vp, vp, vp, i32, i32, vp, i32, vp]
    L.orc_mx_expert.argtypes = [i32, i32, vp, C.POINTER(MxExpertW), vp, i32, vp, vp]
    L.orc_mx_layer.argtypes = [i32, i32, i32, i32, i32, f32, vp, vp, vp,
                               C.POINTER(MxExpertW), C.POINTER(MxExpertW), vp, i32, vp, vp, vp]
    L.orc_cache_sim.argtypes = [i32, i32, i32, i32, i32, vp, vp, i32, i32,
                                C.POINTER(CacheEvent), C.c_int64, C.POINTER(CacheStats)]
    L.orc_cache_sim.restype = C.c_int64
    L.orc_lookahead.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp]
    L.orc_lookahead.restype = None
    L.orc_residual_bf16.argtypes = [i32, vp, vp, C.c_float, vp]
    L.orc_residual_bf16.restype = None
    L.orc_cache_sim_hot.argtypes = [i32, i32, i32, i32, i32, vp, vp, i32, i32, vp, vp,
                                    C.POINTER(CacheEvent), C.c_int64, C.POINTER(CacheStats), vp]
    L.orc_cache_sim_hot.restype = C.c_int64


def _vp(a):
    return None if a is None else a.ctypes.data


def _c(a, dt):
    a = np.ascontiguousarray(a, dtype=dt)
    return a


# ---- scalar helpers -------------------------------------------------------
def bf16_to_f32(b):
    return lib().orc_bf16_to_f32(int(b))


def f16_to_f32(h):
    return lib().orc_f16_to_f32(int(h))


def f32_to_bf16(f):
    return lib().orc_f32_to_bf16(float(f))


def e2m1_value(c):
    return lib().orc_e2m1_value(int(c))


def e8m0_value(e):
    return lib().orc_e8m0_value(int(e))


# ---- array entry points ---------------------------------------------------
def quant_row(v):
    v = _c(v, np.float32)
    q = np.empty(v.shape[0], np.int8)
    s = np.zeros(1, np.float32)
    lib().orc_quant_row(_vp(v), v.shape[0], _vp(q), _vp(s))
    return q, float(s[0])


def quant_rows(x):
    """Row-wise quant of a [T,K] fp32 array -> (q [T,K] int8, s [T] fp32)."""
    x = _c(x, np.float32)
    q = np.empty(x.shape, np.int8)
    s = np.empty(x.shape[0], np.float32)
    for t in range(x.shape[0]):
        q[t], s[t] = quant_row(x[t])
    return q, s


def router(x_bf16, Wr, b, k, r, want=False):
    x_bf16 = _c(x_bf16, np.uint16)
    Wr = _c(Wr, np.float32)
    b = _c(b, np.float32)
    T, H = x_bf16.shape
    E = Wr.shape[0]
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    lg = sc = ch = None
    if want:
        lg = np.empty((T, E), np.float64)
        sc = np.empty((T, E), np.float64)
        ch = np.empty((T, E), np.float64)
    lib().orc_router(T, H, E, k, float(r), _vp(x_bf16), _vp(Wr), _vp(b),
                     _vp(idx), _vp(w), _vp(lg), _vp(sc), _vp(ch))
    if want:
        return idx, w, lg, sc, ch
    return idx, w


def proj_i4i8(q_in, s_in, qw, S, g, rows=None):
    q_in = _c(q_in, np.int8)
    qw = _c(qw, np.int8)
    S = _c(S, np.uint16)
    N, K = qw.shape
    rr = None if rows is None else _c(rows, np.int32)
    cnt = N if rr is None else rr.shape[0]
    y = np.empty(cnt, np.float32)
    lib().orc_proj_i4i8(_vp(q_in), float(s_in), _vp(qw), _vp(S), N, K, g,
                        _vp(rr), 0 if rr is None else cnt, _vp(y))
    return y


def group_dots(q_in, qw, g):
    q_in = _c(q_in, np.int8)
    qw = _c(qw, np.int8)
    N, K = qw.shape
    acc = np.empty((N, K // g), np.int32)
    lib().orc_group_dots(_vp(q_in), _vp(qw), N, K, g, _vp(acc))
    return acc


def rows_exact_fp64(S, K, g):
    S = _c(S, np.uint16)
    return bool(lib().orc_rows_exact_fp64(_vp(S), S.shape[0], K, g))


class _Keep:
    """Holds numpy arrays alive while a ctypes struct points at them."""

    def __init__(self):
        self.refs = []

    def arr(self, a, dt):
        a = _c(a, dt)
        self.refs.append(a)
        return a.ctypes.data


def expert_struct(ex, keep):
    """ex: dict with q_gate,s_gate,q_up,s_up,q_down,s_down numpy arrays."""
    return ExpertW(keep.arr(ex["q_gate"], np.int8), keep.arr(ex["s_gate"], np.uint16),
                   keep.arr(ex["q_up"], np.int8), keep.arr(ex["s_up"], np.uint16),
                   keep.arr(ex["q_down"], np.int8), keep.arr(ex["s_down"], np.uint16))


def mx_expert_struct(ex, keep):
    return MxExpertW(keep.arr(ex["c_gate"], np.uint8), keep.arr(ex["e_gate"], np.uint8),
                     keep.arr(ex["c_up"], np.uint8), keep.arr(ex["e_up"], np.uint8),
                     keep.arr(ex["c_down"], np.uint8), keep.arr(ex["e_down"], np.uint8))


def expert(qa, sa, ex, g, down_rows=None):
    """Returns dict(y, h, qh, sh) for one quantised token row."""
    keep = _Keep()
    w = expert_struct(ex, keep)
    qa = _c(qa, np.int8)
    F, H = ex["q_gate"].shape
    rr = None if down_rows is None else _c(down_rows, np.int32)
    cnt = H if rr is None else rr.shape[0]
    y = np.empty(cnt, np.float32)
    h = np.empty(F, np.float32)
    qh = np.empty(F, np.int8)
    sh = np.zeros(1, np.float32)
    lib().orc_expert(H, F, g, _vp(qa), float(sa), C.byref(w), _vp(rr),
                     0 if rr is None else cnt, _vp(y), _vp(h), _vp(qh), _vp(sh))
    return dict(y=y, h=h, qh=qh, sh=float(sh[0]))


def layer(x_bf16, Wr, b, experts, shared, k, r, g, out_rows=None, expert_map=None):
    """Full int4 layer.  experts: list of expert dicts (or a list of distinct
    expert dicts plus expert_map[e] -> index into it).  Returns (idx, w, out)."""
    x_bf16 = _c(x_bf16, np.uint16)
    Wr = _c(Wr, np.float32)
    b = _c(b, np.float32)
    T, H = x_bf16.shape
    E = Wr.shape[0]
    keep = _Keep()
    distinct = [expert_struct(ex, keep) for ex in experts]
    emap = list(range(E)) if expert_map is None else list(expert_map)
    arr = (ExpertW * E)(*[distinct[emap[e]] for e in range(E)])
    F = experts[0]["q_gate"].shape[0]
    sh = expert_struct(shared, keep) if shared is not None else None
    rr = None if out_rows is None else _c(out_rows, np.int32)
    cnt = H if rr is None else rr.shape[0]
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    out = np.empty((T, cnt), np.float32)
    lib().orc_layer(T, H, F, E, k, g, float(r), _vp(x_bf16), _vp(Wr), _vp(b),
                    arr, C.byref(sh) if sh is not None else None,
                    _vp(rr), 0 if rr is None else cnt, _vp(idx), _vp(w), _vp(out))
    return idx, w, out


def proj_mx(a, codes, e8m0, rows=None):
    a = _c(a, np.float32)
    codes = _c(codes, np.uint8)
    e8m0 = _c(e8m0, np.uint8)
    N, K = codes.shape
    rr = None if rows is None else _c(rows, np.int32)
    cnt = N if rr is None else rr.shape[0]
    y = np.empty(cnt, np.float32)
    lib().orc_proj_mx(_vp(a), _vp(codes), _vp(e8m0), N, K, _vp(rr),
                      0 if rr is None else cnt, _vp(y))
    return y


def mx_expert(a, ex, down_rows=None):
    keep = _Keep()
    w = mx_expert_struct(ex, keep)
    a = _c(a, np.float32)
    F, H = ex["c_gate"].shape
    rr = None if down_rows is None else _c(down_rows, np.int32)
    cnt = H if rr is None else rr.shape[0]
    y = np.empty(cnt, np.float32)
    hb = np.empty(F, np.uint16)
    lib().orc_mx_expert(H, F, _vp(a), C.byref(w), _vp(rr), 0 if rr is None else cnt,
                        _vp(y), _vp(hb))
    return dict(y=y, h_bf16=hb)


def mx_layer(x_bf16, Wr, b, experts, shared, k, r, out_rows=None, expert_map=None):
    x_bf16 = _c(x_bf16, np.uint16)
    Wr = _c(Wr, np.float32)
    b = _c(b, np.float32)
    T, H = x_bf16.shape
    E = Wr.shape[0]
    keep = _Keep()
    distinct = [mx_expert_struct(ex, keep) for ex in experts]
    emap = list(range(E)) if expert_map is None else list(expert_map)
    arr = (MxExpertW * E)(*[distinct[emap[e]] for e in range(E)])
    F = experts[0]["c_gate"].shape[0]
    sh = mx_expert_struct(shared, keep) if shared is not None else None
    rr = None if out_rows is None else _c(out_rows, np.int32)
    cnt = H if rr is None else rr.shape[0]
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    out = np.empty((T, cnt), np.float32)
    lib().orc_mx_layer(T, H, F, E, k, float(r), _vp(x_bf16), _vp(Wr), _vp(b),
                       arr, C.byref(sh) if sh is not None else None,
                       _vp(rr), 0 if rr is None else cnt, _vp(idx), _vp(w), _vp(out))
    return idx, w, out


def cache_sim(L, E, k, n_slots, demand, predict=None, wrap=True, per_layer=False):
    """demand: [steps, L, k] int32.  predict: same shape or None.
    Returns (events [n,4] int32 array (kind, layer, expert, slot), stats dict)
    or raises on capacity failure."""
    demand = _c(demand, np.int32)
    steps = demand.shape[0]
    pr = None if predict is None else _c(predict, np.int32)
    cap = steps * L * k * 4 + 16
    ev = (CacheEvent * cap)()
    st = CacheStats()
    n = lib().orc_cache_sim(L, E, k, n_slots, steps, _vp(demand), _vp(pr),
                            1 if wrap else 0, 1 if per_layer else 0, ev, cap, C.byref(st))
    if n < 0:
        raise RuntimeError("cache simulation failed (capacity below k?)")
    out = np.frombuffer(ev, dtype=np.int32, count=4 * n).reshape(n, 4).copy()
    stats = {f: getattr(st, f) for f, _ in CacheStats._fields_}
    return out, stats


def cache_sim_hot(L, E, k, n_slots, demand, predict=None, wrap=True, per_layer=False,
                  usage_init=None, pin_before=None):
    """The replay with the learned pinned hot-store.  pin_before: [steps] int32,
    the PIN(n) done before each step (-1: none), or None.  Returns (events,
    stats, usage [L*E] int64)."""
    demand = _c(demand, np.int32)
    steps = demand.shape[0]
    pr = None if predict is None else _c(predict, np.int32)
    ui = None if usage_init is None else _c(usage_init, np.int64)
    pb = None if pin_before is None else _c(pin_before, np.int32)
    cap = steps * L * k * 4 + 16 + (0 if pb is None else 2 * int(np.maximum(pb, 0).sum()))
    ev = (CacheEvent * cap)()
    st = CacheStats()
    usage = np.zeros(L * E, np.int64)
    n = lib().orc_cache_sim_hot(L, E, k, n_slots, steps, _vp(demand), _vp(pr),
                                1 if wrap else 0, 1 if per_layer else 0, _vp(ui), _vp(pb),
                                ev, cap, C.byref(st), _vp(usage))
    if n < 0:
        raise RuntimeError("cache simulation failed (capacity below k?)")
    out = np.frombuffer(ev, dtype=np.int32, count=4 * n).reshape(n, 4).copy()
    stats = {f: getattr(st, f) for f, _ in CacheStats._fields_}
    return out, stats, usage


def lookahead(x_bf16, Wr_next, b_next, k):
    """Predicted experts [T,k] of the next layer from the current state."""
    x_bf16 = _c(x_bf16, np.uint16)
    Wr_next = _c(Wr_next, np.float32)
    b_next = _c(b_next, np.float32)
    T, H = x_bf16.shape
    idx = np.empty((T, k), np.int32)
    lib().orc_lookahead(T, H, Wr_next.shape[0], k, _vp(x_bf16), _vp(Wr_next), _vp(b_next),
                        _vp(idx))
    return idx


def residual_bf16(x_bf16, y, gamma):
    """bf16(fp32(x) + fp32(gamma * y)) elementwise."""
    x_bf16 = _c(x_bf16, np.uint16)
    y = _c(y, np.float32)
    out = np.empty_like(x_bf16)
    lib().orc_residual_bf16(x_bf16.size, _vp(x_bf16), _vp(y), float(gamma), _vp(out))
    return out
