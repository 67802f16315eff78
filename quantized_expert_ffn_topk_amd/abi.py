"""ctypes binding of libmoe.so (include/moe.h), same names as the C ABI.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Device buffers may be given as torch tensors (their data_ptr() is
passed), as integers (raw addresses) or as None (NULL).  Streams are torch
streams, raw hipStream_t integers or None (the null stream).  A non-OK status
raises MoEError carrying moe_last_error().
"""
import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB: another build of the same library (an instrumented host build, an
# A/B variant); the in-tree libmoe.so otherwise
LIB_PATH = os.environ.get("MOE_LIB") or os.path.join(PKG, "libmoe.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")

OK, E_INVAL, E_UNSUPPORTED, E_NOMEM, E_HIP, E_CAPACITY = range(6)
WFMT_INT4, WFMT_MXFP4 = 0, 1
DT_F32, DT_BF16 = 0, 1
PATH_AUTO, PATH_GEMV, PATH_MFMA, PATH_MX_BF16 = 0, 1, 2, 3
CACHE_GLOBAL_LRU, CACHE_PER_LAYER_LRU = 0, 1
CACHE_BACKEND_HIP, CACHE_BACKEND_HOST = 0, 1
STAGE_DEMAND, STAGE_PREFETCH, STAGE_PREFETCH_IDLE = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024

_NAMES = {OK: "OK", E_INVAL: "E_INVAL", E_UNSUPPORTED: "E_UNSUPPORTED", E_NOMEM: "E_NOMEM",
          E_HIP: "E_HIP", E_CAPACITY: "E_CAPACITY"}


class MoEError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (_NAMES.get(status, status), msg))
        self.status = status


class moe_layer_desc(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("ffn", C.c_int32), ("n_experts", C.c_int32),
                ("top_k", C.c_int32), ("n_shared", C.c_int32), ("group", C.c_int32),
                ("routed_scale", C.c_float), ("wfmt", C.c_int32), ("out_dtype", C.c_int32)]


class moe_layer_weights(C.Structure):
    _fields_ = [("router_w", C.c_void_p), ("router_bias", C.c_void_p),
                ("expert_ptrs", C.c_void_p), ("shared", C.c_void_p)]


class moe_cache_desc(C.Structure):
    _fields_ = [("device", C.c_int32), ("n_layers", C.c_int32), ("n_experts", C.c_int32),
                ("blob_bytes", C.c_size_t), ("capacity_bytes", C.c_size_t),
                ("host_blobs", C.c_void_p), ("policy", C.c_int32), ("backend", C.c_int32)]


class moe_cache_stats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in (
        "demand_hits", "demand_misses", "prefetch_issued", "prefetch_used", "prefetch_wasted",
        "prefetch_skipped", "prefetch_resident", "evictions", "bytes_copied", "n_slots",
        "pinned", "pin_fills")] + [("copy_busy_ms", C.c_double), ("copies_timed", C.c_int64)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class moe_cache_event(C.Structure):
    _fields_ = [("kind", C.c_int32), ("layer", C.c_int32), ("expert", C.c_int32),
                ("slot", C.c_int32)]


_lib = None


def lib():
    """The loaded library.  Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe.so is not built (python -m quantized_expert_ffn_topk_amd.build)")
        L = C.CDLL(LIB_PATH)
        _declare(L)
        _lib = L
    return _lib


def _declare(L):
    vp, i32, st = C.c_void_p, C.c_int32, C.c_int32
    P = C.POINTER
    sig = {
        "moe_ctx_create": (st, [i32, P(moe_layer_desc), i32, P(vp)]),
        "moe_ctx_destroy": (None, [vp]),
        "moe_ctx_set_path": (st, [vp, i32]),
        "moe_ctx_profile": (st, [vp, i32]),
        "moe_ctx_profile_read": (st, [vp, P(C.c_double), P(C.c_int64)]),
        "moe_blob_bytes": (C.c_size_t, [P(moe_layer_desc)]),
        "moe_pack_expert_int4": (st, [P(moe_layer_desc), vp, vp, vp, vp, vp, vp, vp]),
        "moe_pack_expert_mxfp4": (st, [P(moe_layer_desc), vp, vp, vp, vp, vp, vp, vp]),
        "moe_router_topk": (st, [vp, vp, i32, P(moe_layer_weights), vp, vp, vp]),
        "moe_expert_ffn": (st, [vp, vp, i32, P(moe_layer_weights), vp, vp, vp, vp]),
        "moe_layer_forward": (st, [vp, vp, i32, P(moe_layer_weights), vp, i32, vp, vp, vp, vp]),
        "moe_layer_forward_noalloc": (st, [P(moe_layer_desc), vp, i32, P(moe_layer_weights), vp,
                                           vp, vp, vp]),
        "moe_cache_create": (st, [P(moe_cache_desc), P(vp)]),
        "moe_cache_destroy": (None, [vp]),
        "moe_cache_stage": (st, [vp, i32, vp, i32, i32, vp, vp]),
        "moe_cache_release": (st, [vp, i32, vp]),
        "moe_cache_table": (vp, [vp, i32]),
        "moe_cache_stats_get": (st, [vp, P(moe_cache_stats)]),
        "moe_cache_reset_stats": (None, [vp]),
        "moe_cache_log_enable": (st, [vp, i32]),
        "moe_cache_event_log": (C.c_int64, [vp, P(moe_cache_event), C.c_int64]),
        "moe_cache_debug_fail_next_copy": (st, [vp]),
        "moe_cache_pin_hot": (st, [vp, i32, i32]),
        "moe_cache_usage_get": (st, [vp, vp]),
        "moe_cache_usage_set": (st, [vp, vp]),
        "moe_host_alloc_pinned": (st, [C.c_size_t, P(vp)]),
        "moe_host_free_pinned": (st, [vp]),
        "moe_last_error": (C.c_char_p, []),
        "moe_debug_read": (st, [vp, i32, vp, C.c_size_t, vp]),
        "moe_debug_project": (st, [vp, vp, i32, vp, vp, i32, vp, vp]),
        "moe_debug_stream_read": (st, [vp, C.c_size_t, vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args


def exported_names():
    """Function names declared in include/moe.h."""
    import re
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


# ---------------------------------------------------------------------------
def addr(x):
    """Device/host address of a tensor, numpy array, int or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):
        return x.ctypes.data
    raise TypeError("cannot take the address of %r" % type(x))


def stream_handle(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def check(status):
    if status != OK:
        raise MoEError(status, lib().moe_last_error().decode(errors="replace"))
    return status


def last_error():
    return lib().moe_last_error().decode(errors="replace")


# ---- thin wrappers with the C names ------------------------------------------
def moe_ctx_create(device, desc, max_tokens):
    h = C.c_void_p()
    check(lib().moe_ctx_create(device, C.byref(desc), max_tokens, C.byref(h)))
    return h.value


def moe_ctx_destroy(ctx):
    lib().moe_ctx_destroy(ctx)


def moe_ctx_set_path(ctx, path):
    check(lib().moe_ctx_set_path(ctx, path))


PROF_NAMES = ["router", "topk", "quant", "permute", "gateup", "requant", "down", "combine",
              "tiles"]


def moe_ctx_profile(ctx, on=True):
    check(lib().moe_ctx_profile(ctx, 1 if on else 0))


def moe_ctx_profile_read(ctx):
    """{kind: (total_ms, launches)} since the last read."""
    n = len(PROF_NAMES)
    ms = (C.c_double * n)()
    cnt = (C.c_int64 * n)()
    check(lib().moe_ctx_profile_read(ctx, ms, cnt))
    return {PROF_NAMES[i]: (ms[i], cnt[i]) for i in range(n)}


def moe_blob_bytes(desc):
    return lib().moe_blob_bytes(C.byref(desc))


def moe_pack_expert_int4(desc, q_gate, s_gate, q_up, s_up, q_down, s_down, blob_host):
    check(lib().moe_pack_expert_int4(C.byref(desc), addr(q_gate), addr(s_gate), addr(q_up),
                                     addr(s_up), addr(q_down), addr(s_down), addr(blob_host)))


def moe_pack_expert_mxfp4(desc, c_gate, e_gate, c_up, e_up, c_down, e_down, blob_host):
    check(lib().moe_pack_expert_mxfp4(C.byref(desc), addr(c_gate), addr(e_gate), addr(c_up),
                                      addr(e_up), addr(c_down), addr(e_down), addr(blob_host)))


def moe_router_topk(ctx, x, T, weights, idx, gate_w, stream=None):
    check(lib().moe_router_topk(ctx, addr(x), T, C.byref(weights), addr(idx), addr(gate_w),
                                stream_handle(stream)))


def moe_expert_ffn(ctx, x, T, weights, idx, gate_w, out, stream=None):
    check(lib().moe_expert_ffn(ctx, addr(x), T, C.byref(weights), addr(idx), addr(gate_w),
                               addr(out), stream_handle(stream)))


def moe_layer_forward(ctx, x, T, weights, cache, layer, idx_out, gate_w_out, out, stream=None):
    check(lib().moe_layer_forward(ctx, addr(x), T, C.byref(weights), cache, layer,
                                  addr(idx_out), addr(gate_w_out), addr(out),
                                  stream_handle(stream)))


def moe_layer_forward_noalloc(desc, x, T, weights, idx_out, gate_w_out, out, stream=None):
    check(lib().moe_layer_forward_noalloc(C.byref(desc), addr(x), T, C.byref(weights),
                                          addr(idx_out), addr(gate_w_out), addr(out),
                                          stream_handle(stream)))


def moe_cache_create(desc):
    h = C.c_void_p()
    check(lib().moe_cache_create(C.byref(desc), C.byref(h)))
    return h.value


def moe_cache_destroy(cache):
    lib().moe_cache_destroy(cache)


def moe_cache_stage(cache, layer, ids_host, mode, compute=None, want_ptrs=False):
    import numpy as np
    ids = np.ascontiguousarray(ids_host, dtype=np.int32)
    ptrs = (C.c_void_p * max(1, len(ids)))() if want_ptrs else None
    check(lib().moe_cache_stage(cache, layer, ids.ctypes.data, len(ids), mode,
                                stream_handle(compute), ptrs))
    return [p for p in ptrs[:len(ids)]] if want_ptrs else None


def moe_cache_release(cache, layer, compute=None):
    check(lib().moe_cache_release(cache, layer, stream_handle(compute)))


def moe_cache_table(cache, layer):
    return lib().moe_cache_table(cache, layer)


def moe_cache_stats_get(cache):
    s = moe_cache_stats()
    check(lib().moe_cache_stats_get(cache, C.byref(s)))
    return s.as_dict()


def moe_cache_reset_stats(cache):
    lib().moe_cache_reset_stats(cache)


def moe_cache_log_enable(cache, on=True):
    check(lib().moe_cache_log_enable(cache, 1 if on else 0))


def moe_cache_event_log(cache, cap=1 << 20):
    import numpy as np
    buf = (moe_cache_event * cap)()
    n = lib().moe_cache_event_log(cache, buf, cap)
    if n < 0:
        raise MoEError(E_INVAL, "event log read failed")
    return np.frombuffer(buf, dtype=np.int32, count=4 * n).reshape(n, 4).copy()


def moe_cache_debug_fail_next_copy(cache):
    check(lib().moe_cache_debug_fail_next_copy(cache))


def moe_cache_pin_hot(cache, n, reserve):
    check(lib().moe_cache_pin_hot(cache, n, reserve))


def moe_cache_usage_get(cache, n_keys):
    import numpy as np
    u = np.zeros(n_keys, np.int64)
    check(lib().moe_cache_usage_get(cache, u.ctypes.data))
    return u


def moe_cache_usage_set(cache, usage):
    import numpy as np
    u = np.ascontiguousarray(usage, np.int64)
    check(lib().moe_cache_usage_set(cache, u.ctypes.data))


def moe_host_alloc_pinned(nbytes):
    p = C.c_void_p()
    check(lib().moe_host_alloc_pinned(nbytes, C.byref(p)))
    return p.value


def moe_host_free_pinned(p):
    check(lib().moe_host_free_pinned(p))


def moe_last_error():
    return last_error()


def moe_debug_read(ctx, which, dst, nbytes, stream=None):
    check(lib().moe_debug_read(ctx, which, addr(dst), nbytes, stream_handle(stream)))


def moe_debug_project(ctx, blob, part, q_in, s_in, T, y, stream=None):
    check(lib().moe_debug_project(ctx, addr(blob), part, addr(q_in), addr(s_in), T, addr(y),
                                  stream_handle(stream)))


def moe_debug_stream_read(src, nbytes, sink, stream=None):
    check(lib().moe_debug_stream_read(addr(src), nbytes, addr(sink), stream_handle(stream)))
