"""CPU tests of libmoe.so: exports, argument validation, the packer, and the
cache's logical state machine (host backend) against the oracle simulator.
No test here launches a kernel."""
import ctypes as C
import json
import os

import numpy as np
import pytest

from quantized_expert_ffn_topk_amd import abi, synth
from quantized_expert_ffn_topk_amd.layer import make_desc, pack_int4, pack_mxfp4

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def L():
    return abi.lib()


def test_every_header_symbol_is_exported(L):
    names = abi.exported_names()
    assert len(names) >= 24
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


@pytest.mark.parametrize("H,F,g,wfmt,want", [
    (6144, 2048, 32, abi.WFMT_INT4, 21233664),
    (2048, 1024, 32, abi.WFMT_INT4, 3538944),
    (6144, 2048, 64, abi.WFMT_INT4, 20054016),
    (7168, 2048, 32, abi.WFMT_MXFP4, 23396352),
])
def test_blob_bytes(H, F, g, wfmt, want):
    d = make_desc(H, F, 8, 2, 1, g, 1.0, wfmt)
    assert abi.moe_blob_bytes(d) == want


def test_blob_bytes_match_page_figures():
    gold = json.load(open(os.path.join(HERE, "golden", "page_figures.json")))
    shp = gold["glm_expert_shape"]
    d = make_desc(shp["hidden"], shp["ffn"], 256, 8, 1, 64)
    b = abi.moe_blob_bytes(d)
    e = gold["expert_bytes_approx"]
    assert abs(b - e["value"]) <= e["tolerance_rel"] * e["value"]
    c = gold["cold_token_bytes_approx"]
    tot = b * c["layers"] * c["experts_per_layer"]
    assert abs(tot - c["value"]) <= c["tolerance_rel"] * c["value"]


@pytest.mark.parametrize("field,val", [
    ("hidden", 100), ("ffn", 0), ("n_experts", 0), ("n_experts", 2000), ("top_k", 0),
    ("top_k", 33), ("n_shared", 2), ("group", 16), ("wfmt", 7), ("out_dtype", 5)])
def test_invalid_desc_rejected_before_any_gpu_call(field, val):
    d = make_desc(256, 256, 8, 2, 1)
    setattr(d, field, val)
    assert abi.moe_blob_bytes(d) == 0
    with pytest.raises(abi.MoEError) as ei:
        abi.moe_ctx_create(0, d, 4)
    assert ei.value.status == abi.E_INVAL


def test_topk_above_experts_rejected():
    d = make_desc(256, 256, 4, 5, 0)
    with pytest.raises(abi.MoEError) as ei:
        abi.moe_ctx_create(0, d, 4)
    assert ei.value.status == abi.E_INVAL


def test_null_ctx_calls_fail_cleanly(L):
    w = abi.moe_layer_weights()
    assert L.moe_router_topk(None, None, 1, C.byref(w), None, None, None) == abi.E_INVAL
    assert L.moe_expert_ffn(None, None, 1, C.byref(w), None, None, None, None) == abi.E_INVAL
    assert L.moe_layer_forward(None, None, 1, C.byref(w), None, 0, None, None, None, None) == abi.E_INVAL
    assert "NULL" in abi.last_error()


# ---------------------------------------------------------------------------
# packer
# ---------------------------------------------------------------------------
def unpack_int4(blob, H, F, g):
    """Reads a blob back following the documented layout."""
    def tiles(off, n_tiles, K, rows_of_tile):
        KC = K // 32
        q = {}
        for t in range(n_tiles):
            base = off + t * K * 8
            chunk = blob[base:base + K * 8].reshape(KC, 16, 16)
            lo = ((chunk & 15).astype(np.int16) ^ 8) - 8     # 4-bit two's complement
            hi = ((chunk >> 4).astype(np.int16) ^ 8) - 8
            vals = np.concatenate([lo, hi], axis=2)          # [KC, r, 32]
            q[t] = vals.transpose(1, 0, 2).reshape(16, K)
        return q

    def scales(off, n_tiles, K):
        G = K // g
        s = {}
        for t in range(n_tiles):
            base = off + t * G * 16 * 2
            s[t] = blob[base:base + G * 32].view(np.uint16).reshape(G, 16).T
        return s

    gu_w = 0
    gu_s = F * H
    dn_w = gu_s + (F // 8) * (H // g) * 32
    dn_s = dn_w + (H // 16) * F * 8
    qgu = tiles(gu_w, F // 8, H, None)
    sgu = scales(gu_s, F // 8, H)
    qdn = tiles(dn_w, H // 16, F, None)
    sdn = scales(dn_s, H // 16, F)
    qg = np.concatenate([qgu[2 * b] for b in range(F // 16)])
    qu = np.concatenate([qgu[2 * b + 1] for b in range(F // 16)])
    sg = np.concatenate([sgu[2 * b] for b in range(F // 16)])
    su = np.concatenate([sgu[2 * b + 1] for b in range(F // 16)])
    qd = np.concatenate([qdn[t] for t in range(H // 16)])
    sd = np.concatenate([sdn[t] for t in range(H // 16)])
    return dict(q_gate=qg, s_gate=sg, q_up=qu, s_up=su, q_down=qd, s_down=sd)


@pytest.mark.parametrize("g", [32, 64])
def test_pack_int4_round_trip(g):
    H, F = 512, 256
    ex = synth.expert_int4(3, 0, H, F, g)
    d = make_desc(H, F, 4, 2, 0, g)
    blob = pack_int4(d, ex)
    assert blob.nbytes == abi.moe_blob_bytes(d)
    back = unpack_int4(blob, H, F, g)
    for k in ex:
        assert np.array_equal(back[k].astype(ex[k].dtype), ex[k]), k


def test_pack_rejects_bad_codes_and_scales():
    H, F, g = 256, 256, 32
    d = make_desc(H, F, 4, 2, 0, g)
    ex = synth.expert_int4(4, 0, H, F, g)
    bad = dict(ex)
    bad["q_up"] = ex["q_up"].copy()
    bad["q_up"][3, 5] = 8
    with pytest.raises(abi.MoEError) as ei:
        pack_int4(d, bad)
    assert ei.value.status == abi.E_INVAL
    bad = dict(ex)
    bad["s_down"] = ex["s_down"].copy()
    bad["s_down"][1, 1] = 0x7E00            # fp16 NaN
    with pytest.raises(abi.MoEError):
        pack_int4(d, bad)
    bad = dict(ex)
    s = ex["s_gate"].copy().view(np.float16)
    s[0, 0] = np.float16(6e-8)
    s[0, 1] = np.float16(60000.0)           # ~40 binades apart in one row
    bad["s_gate"] = s.view(np.uint16)
    with pytest.raises(abi.MoEError) as ei:
        pack_int4(d, bad)
    assert "binades" in str(ei.value)


def test_pack_mxfp4_layout_and_nan_scale():
    H, F = 256, 256
    ex = synth.expert_mxfp4(5, 0, H, F)
    d = make_desc(H, F, 4, 2, 0, 32, 1.0, abi.WFMT_MXFP4)
    blob = pack_mxfp4(d, ex)
    # first tile of the gate/up section: gate rows 0..15, chunk 0
    chunk0 = blob[0:16 * 16].reshape(16, 16)
    for r in range(16):
        codes = ex["c_gate"][r, :32]
        want = (codes[0::2] & 15) | ((codes[1::2] & 15) << 4)
        assert np.array_equal(chunk0[r], want.astype(np.uint8))
    # scales of gate tile 0 follow the gate/up weights: [kc][r]
    gu_s = F * H
    sc = blob[gu_s:gu_s + (H // 32) * 16].reshape(H // 32, 16)
    assert np.array_equal(sc.T, ex["e_gate"][:16])
    bad = dict(ex)
    bad["e_down"] = ex["e_down"].copy()
    bad["e_down"][0, 0] = 0xFF
    with pytest.raises(abi.MoEError):
        pack_mxfp4(d, bad)


# ---------------------------------------------------------------------------
# cache state machine, host backend (no GPU) against the oracle simulator
# ---------------------------------------------------------------------------
class HostCache:
    def __init__(self, L_, E, n_slots, per_layer=False, blob=256):
        self.blob = blob
        self.bufs = [np.full(blob, (l * E + e) % 251, np.uint8) for l in range(L_) for e in range(E)]
        for i, b in enumerate(self.bufs):
            b[:8] = np.frombuffer(np.int64(i).tobytes(), np.uint8)
        self.ptrs = (C.c_void_p * len(self.bufs))(*[b.ctypes.data for b in self.bufs])
        d = abi.moe_cache_desc(0, L_, E, blob, blob * n_slots, C.addressof(self.ptrs),
                               abi.CACHE_PER_LAYER_LRU if per_layer else abi.CACHE_GLOBAL_LRU,
                               abi.CACHE_BACKEND_HOST)
        self.h = abi.moe_cache_create(d)
        self.L, self.E = L_, E
        abi.moe_cache_log_enable(self.h, True)

    def slot_key(self, layer, e):
        tab = abi.moe_cache_table(self.h, layer)
        p = C.cast(tab, C.POINTER(C.c_void_p))[e]
        if not p:
            return None
        return int(np.frombuffer(C.string_at(p, 8), np.int64)[0])

    def close(self):
        abi.moe_cache_destroy(self.h)


def run_trace(hc, demand, predict, mode=abi.STAGE_PREFETCH):
    steps, L_, k = demand.shape
    for t in range(steps):
        for l in range(L_):
            abi.moe_cache_stage(hc.h, l, demand[t, l], abi.STAGE_DEMAND)
            for e in demand[t, l]:
                assert hc.slot_key(l, int(e)) == l * hc.E + int(e)   # right blob in the slot
            if predict is not None:
                nl = l + 1
                if nl == L_:
                    nl = 0
                    if t + 1 >= steps:
                        abi.moe_cache_release(hc.h, l)
                        continue
                abi.moe_cache_stage(hc.h, nl, predict[t, l], mode)
            abi.moe_cache_release(hc.h, l)


@pytest.mark.parametrize("cap,per_layer,with_pred", [
    (8, False, False), (13, False, True), (24, False, True), (40, True, True), (64, False, True)])
def test_host_cache_log_equals_oracle_sim(orc, cap, per_layer, with_pred):
    L_, E, k, steps = 4, 32, 4, 25
    dem, pred = synth.zipf_trace(11, L_, E, k, steps)
    if per_layer and cap // L_ < k:
        pytest.skip("partition below k")
    hc = HostCache(L_, E, cap, per_layer)
    try:
        run_trace(hc, dem, pred if with_pred else None)
        log = abi.moe_cache_event_log(hc.h)
        stats = abi.moe_cache_stats_get(hc.h)
    finally:
        hc.close()
    ev, st = orc.cache_sim(L_, E, k, cap, dem, pred if with_pred else None, wrap=True,
                           per_layer=per_layer)
    assert np.array_equal(log, ev)
    for key in st:
        assert stats[key] == st[key], key
    assert stats["bytes_copied"] == 256 * (stats["demand_misses"] + stats["prefetch_issued"])


def test_host_cache_idle_prefetch_equals_prefetch(orc):
    # the host backend copies synchronously, so its copy engine is never busy
    # and PREFETCH_IDLE takes every request: the same log as PREFETCH and as
    # the oracle's state machine
    L_, E, k, steps = 4, 32, 4, 25
    dem, pred = synth.zipf_trace(11, L_, E, k, steps)
    hc = HostCache(L_, E, 13, False)
    try:
        run_trace(hc, dem, pred, abi.STAGE_PREFETCH_IDLE)
        log = abi.moe_cache_event_log(hc.h)
        stats = abi.moe_cache_stats_get(hc.h)
    finally:
        hc.close()
    ev, st = orc.cache_sim(L_, E, k, 13, dem, pred, wrap=True, per_layer=False)
    assert np.array_equal(log, ev)
    for key in st:
        assert stats[key] == st[key], key


def test_host_cache_capacity_and_failed_copy():
    hc = HostCache(2, 16, 4)
    try:
        with pytest.raises(abi.MoEError) as ei:
            abi.moe_cache_stage(hc.h, 0, [0, 1, 2, 3, 4], abi.STAGE_DEMAND)
        assert ei.value.status == abi.E_CAPACITY
        assert abi.moe_cache_stats_get(hc.h)["demand_misses"] == 0       # nothing changed
        abi.moe_cache_debug_fail_next_copy(hc.h)
        with pytest.raises(abi.MoEError) as ei:
            abi.moe_cache_stage(hc.h, 0, [5], abi.STAGE_DEMAND)
        assert ei.value.status == abi.E_HIP
        assert hc.slot_key(0, 5) is None                                    # slot left empty
        abi.moe_cache_stage(hc.h, 0, [5], abi.STAGE_DEMAND)                 # retry works
        assert hc.slot_key(0, 5) == 5
        with pytest.raises(abi.MoEError) as ei:
            abi.moe_cache_stage(hc.h, 0, [16], abi.STAGE_DEMAND)
        assert ei.value.status == abi.E_INVAL
        with pytest.raises(abi.MoEError):
            abi.moe_cache_stage(hc.h, 2, [1], abi.STAGE_DEMAND)
        with pytest.raises(abi.MoEError):
            abi.moe_cache_stage(hc.h, 0, [1, 1], abi.STAGE_DEMAND)
    finally:
        hc.close()


@pytest.mark.parametrize("cap,per_layer,n_pin", [(13, False, 5), (24, False, 30), (40, True, 6)])
def test_host_cache_hot_store_equals_oracle_sim(orc, cap, per_layer, n_pin):
    # usage learnt from a history trace (set through moe_cache_usage_set), a
    # first pin before step 0 and a re-pin before step 12 from the counts so
    # far; the event log, the counters and the usage counts equal the oracle's
    L_, E, k, steps = 4, 32, 4, 25
    hist, _ = synth.zipf_trace(12, L_, E, k, steps)
    usage0 = np.bincount((np.arange(L_)[None, :, None] * E + hist).ravel(),
                         minlength=L_ * E).astype(np.int64)
    dem, pred = synth.zipf_trace(11, L_, E, k, steps)
    pin = np.full(steps, -1, np.int32)
    pin[0], pin[12] = n_pin, n_pin
    hc = HostCache(L_, E, cap, per_layer)
    try:
        abi.moe_cache_usage_set(hc.h, usage0)
        for t in range(steps):
            if pin[t] >= 0:
                abi.moe_cache_pin_hot(hc.h, int(pin[t]), k)
            run_trace(hc, dem[t:t + 1], pred[t:t + 1])
        log = abi.moe_cache_event_log(hc.h)
        stats = abi.moe_cache_stats_get(hc.h)
        usage = abi.moe_cache_usage_get(hc.h, L_ * E)
    finally:
        hc.close()
    ev, st, u = orc.cache_sim_hot(L_, E, k, cap, dem, pred, wrap=False, per_layer=per_layer,
                                  usage_init=usage0, pin_before=pin)
    assert np.array_equal(log, ev)
    for key in st:
        assert stats[key] == st[key], key
    assert np.array_equal(usage, u)
    assert stats["pinned"] > 0


def test_host_cache_pin_needs_no_locked_slot_and_valid_usage():
    hc = HostCache(2, 16, 8)
    try:
        abi.moe_cache_stage(hc.h, 0, [1, 2], abi.STAGE_DEMAND)
        with pytest.raises(abi.MoEError) as ei:
            abi.moe_cache_pin_hot(hc.h, 2, 2)                 # layer 0 still holds slots
        assert ei.value.status == abi.E_INVAL
        abi.moe_cache_release(hc.h, 0)
        abi.moe_cache_pin_hot(hc.h, 2, 2)
        assert abi.moe_cache_stats_get(hc.h)["pinned"] == 2
        bad = np.zeros(32, np.int64)
        bad[3] = -1
        with pytest.raises(abi.MoEError):
            abi.moe_cache_usage_set(hc.h, bad)
        assert abi.moe_cache_usage_get(hc.h, 32)[[1, 2]].tolist() == [1, 1]
    finally:
        hc.close()


def test_stream_read_probe_rejects_bad_arguments_before_any_launch():
    # every case returns before a kernel would be enqueued
    for src, n, sink in [(None, 65536, 16), (16, 65536, None), (16, 0, 16), (16, 65536 + 16, 16),
                         (24, 65536, 16)]:
        with pytest.raises(abi.MoEError) as ei:
            abi.moe_debug_stream_read(src, n, sink)
        assert ei.value.status == abi.E_INVAL
