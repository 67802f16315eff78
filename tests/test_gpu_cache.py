"""GPU tests of the HBM expert cache (HIP backend): layers run through the cache
give bit-identical results to all-resident layers whatever the placement, the
logical event log equals the oracle's state machine on the same routing, and a
failed copy (forced from the host) leaves the slot empty and can be retried."""
import ctypes as C

import numpy as np
import pytest

import oracle
from quantized_expert_ffn_topk_amd import abi, synth
from quantized_expert_ffn_topk_amd.layer import Layer, make_desc, pack_int4

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

L_, E, K, H, F = 3, 16, 4, 512, 256


class Stack:
    """L_ layers of E distinct routed experts (+1 shared each) in pinned host
    memory, a cache over them and, for reference, all-resident layers."""

    def __init__(self, n_slots, policy=abi.CACHE_GLOBAL_LRU, max_tokens=1):
        self.desc = make_desc(H, F, E, K, 1, 32, 2.5)
        self.blob = abi.moe_blob_bytes(self.desc)
        self.experts = [[synth.expert_int4(40 + l, e, H, F, 32) for e in range(E)] for l in range(L_)]
        self.shared = [synth.expert_int4(40 + l, -1, H, F, 32) for l in range(L_)]
        self.Wr = [synth.router_weights(40 + l, E, H)[0] for l in range(L_)]
        self.host = abi.moe_host_alloc_pinned(L_ * E * self.blob)
        base = np.ctypeslib.as_array(C.cast(self.host, C.POINTER(C.c_uint8)), shape=(L_ * E * self.blob,))
        for l in range(L_):
            for e in range(E):
                o = (l * E + e) * self.blob
                base[o:o + self.blob] = pack_int4(self.desc, self.experts[l][e])
        self.ptrs = (C.c_void_p * (L_ * E))(*[self.host + i * self.blob for i in range(L_ * E)])
        cd = abi.moe_cache_desc(0, L_, E, self.blob, n_slots * self.blob, C.addressof(self.ptrs),
                                policy, abi.CACHE_BACKEND_HIP)
        self.cache = abi.moe_cache_create(cd)
        abi.moe_cache_log_enable(self.cache, True)
        self.ref = [Layer(self.desc, self.Wr[l], np.zeros(E, np.float32), self.experts[l],
                          self.shared[l], max_tokens=max_tokens) for l in range(L_)]
        self.ctx = abi.moe_ctx_create(0, self.desc, max_tokens)
        self.bias = torch.zeros(E, dtype=torch.float32, device="cuda")
        self.wts = [abi.moe_layer_weights(self.ref[l].Wr.data_ptr(), self.bias.data_ptr(), None,
                                          self.ref[l].shared_blob.data_ptr()) for l in range(L_)]

    def close(self):
        abi.moe_ctx_destroy(self.ctx)
        abi.moe_cache_destroy(self.cache)
        for r in self.ref:
            r.close()
        abi.moe_host_free_pinned(self.host)


def _run(stk, demand, predict, steps, pins=None, mode=abi.STAGE_PREFETCH):
    """The streaming loop: layer l runs through the cache (DEMAND inside the
    forward), then the guess for the next layer is prefetched and layer l is
    released; every output is checked against the resident layer.  pins[t]
    (when >= 0) pins that many hottest keys before step t."""
    used = np.empty_like(demand[:steps])
    idx = torch.empty((1, K), dtype=torch.int32, device="cuda")
    gw = torch.empty((1, K), dtype=torch.float32, device="cuda")
    out = torch.empty((1, H), dtype=torch.float32, device="cuda")
    for t in range(steps):
        if pins is not None and pins[t] >= 0:
            abi.moe_cache_pin_hot(stk.cache, int(pins[t]), K)
        for l in range(L_):
            b = synth.forcing_bias(E, demand[t, l])
            stk.bias.copy_(torch.from_numpy(b))
            x = stk.ref[l].x_tensor(synth.activations(500 + t * L_ + l, 1, H))
            abi.moe_layer_forward(stk.ctx, x, 1, stk.wts[l], stk.cache, l, idx, gw, out)
            stk.ref[l].set_bias(b)
            ri, rw, ro = stk.ref[l].forward(x)
            torch.cuda.synchronize()
            assert np.array_equal(idx.cpu().numpy(), ri.cpu().numpy())
            assert sorted(idx.cpu().numpy()[0].tolist()) == sorted(demand[t, l].tolist())
            assert torch.equal(out.view(torch.int32), ro.view(torch.int32)), (t, l)
            used[t, l] = idx.cpu().numpy()[0]
            if predict is not None:
                nl = l + 1
                if nl == L_:
                    nl = 0
                    if t + 1 >= steps:
                        abi.moe_cache_release(stk.cache, l)
                        continue
                abi.moe_cache_stage(stk.cache, nl, predict[t, l], mode)
            abi.moe_cache_release(stk.cache, l)
    torch.cuda.synchronize()
    return used


@pytest.mark.parametrize("n_slots", [7, 12])
def test_idle_prefetch_keeps_outputs_and_accounts_every_guess(n_slots):
    # PREFETCH_IDLE: which guesses are copied depends on timing, so the log is
    # not compared with the oracle; every output still equals the resident
    # layer's bit for bit (checked in _run), every guessed id is counted once
    # (issued, already resident or skipped), and the events are the known kinds
    steps = 5
    demand, predict = synth.zipf_trace(8, L_, E, K, steps)
    stk = Stack(n_slots)
    try:
        _run(stk, demand, predict, steps, mode=abi.STAGE_PREFETCH_IDLE)
        log = abi.moe_cache_event_log(stk.cache)
        stats = abi.moe_cache_stats_get(stk.cache)
    finally:
        stk.close()
    n_guess = (steps * L_ - 1) * K
    assert stats["prefetch_issued"] + stats["prefetch_resident"] + stats["prefetch_skipped"] == n_guess
    kinds = set(log[:, 0].tolist())
    assert kinds <= {0, 1, 2, 3, 4, 5, 8}
    busy = int((log[:, 0] == 8).sum())
    assert busy <= stats["prefetch_skipped"]
    assert stats["bytes_copied"] == stk.blob * (stats["demand_misses"] + stats["prefetch_issued"])
    print("idle prefetch, %d slots: %d issued, %d resident, %d skipped (%d with the copy engine "
          "busy)" % (n_slots, stats["prefetch_issued"], stats["prefetch_resident"],
                     stats["prefetch_skipped"], busy))


@pytest.mark.parametrize("n_slots,with_pred", [(6, False), (9, True), (24, True)])
def test_cached_layers_equal_resident_layers_and_oracle_log(n_slots, with_pred):
    steps = 5
    demand, predict = synth.zipf_trace(7, L_, E, K, steps)
    stk = Stack(n_slots)
    try:
        used = _run(stk, demand, predict if with_pred else None, steps)
        log = abi.moe_cache_event_log(stk.cache)
        stats = abi.moe_cache_stats_get(stk.cache)
    finally:
        stk.close()
    ev, st = oracle.cache_sim(L_, E, K, n_slots, used, predict[:steps] if with_pred else None,
                              wrap=True)
    assert np.array_equal(log, ev)
    for key in st:
        assert stats[key] == st[key], key
    assert stats["bytes_copied"] == stk.blob * (stats["demand_misses"] + stats["prefetch_issued"])
    # every copy was timed, and the copy engine's busy time is positive
    assert stats["copies_timed"] == stats["demand_misses"] + stats["prefetch_issued"]
    assert stats["copy_busy_ms"] > 0.0


def _project(ctx, blob, q):
    """Gate and up projections of one int8 row through `blob` (unit scale)."""
    ys = []
    ones = torch.ones(1, dtype=torch.float32, device="cuda")
    for part in (0, 1):
        y = torch.empty((1, F), dtype=torch.float32, device="cuda")
        abi.moe_debug_project(ctx, blob, part, q, ones, 1, y)
        ys.append(y)
    torch.cuda.synchronize()
    return torch.cat(ys, 1)


def test_failed_copy_leaves_slot_empty_and_retry_works():
    stk = Stack(8)
    try:
        abi.moe_cache_debug_fail_next_copy(stk.cache)
        with pytest.raises(abi.MoEError) as ei:
            abi.moe_cache_stage(stk.cache, 1, [3], abi.STAGE_DEMAND)
        assert ei.value.status == abi.E_HIP
        st = abi.moe_cache_stats_get(stk.cache)
        assert st["bytes_copied"] == 0
        # the retry copies the blob of (layer 1, expert 3) into a slot: the
        # slot's gate/up projections equal those of the resident blob
        p = abi.moe_cache_stage(stk.cache, 1, [3], abi.STAGE_DEMAND, want_ptrs=True)[0]
        assert p
        q = torch.from_numpy(np.random.default_rng(5).integers(-127, 128, size=(1, H)).astype(np.int8)).cuda()
        got = _project(stk.ctx, p, q)
        want = _project(stk.ctx, stk.ref[1].blobs[3].data_ptr(), q)
        assert torch.equal(got.view(torch.int32), want.view(torch.int32))
        abi.moe_cache_release(stk.cache, 1)
    finally:
        stk.close()


@pytest.mark.parametrize("layer", [-1, L_])
def test_layer_forward_rejects_layer_out_of_range_before_enqueue(layer):
    # a layer index outside [0, n_layers) is an argument error caught before
    # the router is enqueued: the caller's idx / gate_w / out stay untouched
    stk = Stack(8)
    try:
        idx = torch.full((1, K), -7, dtype=torch.int32, device="cuda")
        gw = torch.full((1, K), -7.0, dtype=torch.float32, device="cuda")
        out = torch.full((1, H), -7.0, dtype=torch.float32, device="cuda")
        x = stk.ref[0].x_tensor(synth.activations(9, 1, H))
        with pytest.raises(abi.MoEError) as ei:
            abi.moe_layer_forward(stk.ctx, x, 1, stk.wts[0], stk.cache, layer, idx, gw, out)
        assert ei.value.status == abi.E_INVAL
        torch.cuda.synchronize()
        assert bool((idx == -7).all()) and bool((gw == -7.0).all()) and bool((out == -7.0).all())
        assert abi.moe_cache_stats_get(stk.cache)["bytes_copied"] == 0
    finally:
        stk.close()


@pytest.mark.parametrize("n_slots,n_pin", [(9, 4), (14, 8)])
def test_hot_store_pins_equal_oracle_and_keep_placement_invariance(n_slots, n_pin):
    # usage from an earlier session of the same routing model, pins before
    # step 0 and again before step 3; outputs stay bit-identical to the
    # resident layers, and the event log, counters and usage equal the
    # oracle's hot-store replay
    steps = 6
    hist, _ = synth.zipf_trace(17, L_, E, K, 12, model_seed=7)
    usage0 = np.bincount((np.arange(L_)[None, :, None] * E + hist).ravel(),
                         minlength=L_ * E).astype(np.int64)
    demand, predict = synth.zipf_trace(7, L_, E, K, steps)
    pins = np.full(steps, -1, np.int32)
    pins[0], pins[3] = n_pin, n_pin
    stk = Stack(n_slots)
    try:
        abi.moe_cache_usage_set(stk.cache, usage0)
        used = _run(stk, demand, predict, steps, pins)
        log = abi.moe_cache_event_log(stk.cache)
        stats = abi.moe_cache_stats_get(stk.cache)
        usage = abi.moe_cache_usage_get(stk.cache, L_ * E)
    finally:
        stk.close()
    ev, st, u = oracle.cache_sim_hot(L_, E, K, n_slots, used, predict[:steps], wrap=True,
                                     usage_init=usage0, pin_before=pins)
    assert np.array_equal(log, ev)
    for key in st:
        assert stats[key] == st[key], key
    assert np.array_equal(usage, u)
    assert stats["pinned"] == min(n_pin, n_slots - K)
    assert stats["bytes_copied"] == stk.blob * (stats["demand_misses"] + stats["prefetch_issued"] +
                                                stats["pin_fills"])


def test_multi_token_calls_through_the_cache_equal_resident_layers():
    # three tokens per call (the few-token GEMV path reading the slots): the
    # cache stages every distinct expert of the call, the outputs equal the
    # all-resident layer's bit for bit; a call needing more slots than the
    # pool has fails with E_CAPACITY, leaves the cache as it was, and a
    # one-token call goes through afterwards
    T = 3
    stk = Stack(16, max_tokens=T)
    small = Stack(6, max_tokens=T)
    try:
        idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
        gw = torch.empty((T, K), dtype=torch.float32, device="cuda")
        out = torch.empty((T, H), dtype=torch.float32, device="cuda")
        for t in range(3):
            for l in range(L_):
                x = stk.ref[l].x_tensor(synth.activations(800 + t * L_ + l, T, H))
                abi.moe_layer_forward(stk.ctx, x, T, stk.wts[l], stk.cache, l, idx, gw, out)
                ri, rw, ro = stk.ref[l].forward(x)
                torch.cuda.synchronize()
                assert np.array_equal(idx.cpu().numpy(), ri.cpu().numpy()), (t, l)
                assert torch.equal(gw.view(torch.int32), rw.view(torch.int32)), (t, l)
                assert torch.equal(out.view(torch.int32), ro.view(torch.int32)), (t, l)
                abi.moe_cache_release(stk.cache, l)
        # six slots: a call whose three tokens pick more than six experts
        failed = 0
        for s_ in range(6):
            x = small.ref[0].x_tensor(synth.activations(900 + s_, T, H))
            ri, _, _ = small.ref[0].forward(x)
            torch.cuda.synchronize()
            need = len(set(ri.cpu().numpy().ravel().tolist()))
            before = abi.moe_cache_stats_get(small.cache)
            if need > 6:
                with pytest.raises(abi.MoEError) as ei:
                    abi.moe_layer_forward(small.ctx, x, T, small.wts[0], small.cache, 0, idx, gw, out)
                assert ei.value.status == abi.E_CAPACITY
                assert abi.moe_cache_stats_get(small.cache)["bytes_copied"] == before["bytes_copied"]
                failed += 1
            else:
                abi.moe_layer_forward(small.ctx, x, T, small.wts[0], small.cache, 0, idx, gw, out)
                abi.moe_cache_release(small.cache, 0)
        assert failed > 0
        one_i = torch.empty((1, K), dtype=torch.int32, device="cuda")
        one_w = torch.empty((1, K), dtype=torch.float32, device="cuda")
        one_o = torch.empty((1, H), dtype=torch.float32, device="cuda")
        x1 = small.ref[0].x_tensor(synth.activations(950, 1, H))
        abi.moe_layer_forward(small.ctx, x1, 1, small.wts[0], small.cache, 0, one_i, one_w, one_o)
        ri, rw, ro = small.ref[0].forward(x1)
        torch.cuda.synchronize()
        assert torch.equal(one_o.view(torch.int32), ro.view(torch.int32))
        abi.moe_cache_release(small.cache, 0)
    finally:
        stk.close()
        small.close()


def test_mxfp4_layer_through_the_cache_equals_resident():
    # MXFP4 blobs staged like int4 ones: one- and two-token calls through the
    # cache give the resident layer's bits (same kernels on the same bytes,
    # only the placement differs)
    from quantized_expert_ffn_topk_amd.layer import pack_mxfp4
    Tm = 2
    desc = make_desc(H, F, E, K, 1, 32, 1.0, abi.WFMT_MXFP4)
    blob = abi.moe_blob_bytes(desc)
    experts = [synth.expert_mxfp4(60, e, H, F) for e in range(E)]
    shared = synth.expert_mxfp4(60, -1, H, F)
    Wr, _ = synth.router_weights(60, E, H)
    bias = synth.uniform_bias(60, E)
    host = abi.moe_host_alloc_pinned(E * blob)
    ref = None
    cache = None
    ctx = None
    try:
        base = np.ctypeslib.as_array(C.cast(host, C.POINTER(C.c_uint8)), shape=(E * blob,))
        for e in range(E):
            base[e * blob:(e + 1) * blob] = pack_mxfp4(desc, experts[e])
        ptrs = (C.c_void_p * E)(*[host + e * blob for e in range(E)])
        cd = abi.moe_cache_desc(0, 1, E, blob, 10 * blob, C.addressof(ptrs), abi.CACHE_GLOBAL_LRU,
                                abi.CACHE_BACKEND_HIP)
        cache = abi.moe_cache_create(cd)
        ref = Layer(desc, Wr, bias, experts, shared, max_tokens=Tm)
        ctx = abi.moe_ctx_create(0, desc, Tm)
        bz = torch.from_numpy(bias).to("cuda")
        wts = abi.moe_layer_weights(ref.Wr.data_ptr(), bz.data_ptr(), None, ref.shared_blob.data_ptr())
        for T in (1, 2):
            idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
            gw = torch.empty((T, K), dtype=torch.float32, device="cuda")
            out = torch.empty((T, H), dtype=torch.float32, device="cuda")
            for s_ in range(4):
                x = ref.x_tensor(synth.activations(700 + 10 * T + s_, T, H))
                abi.moe_layer_forward(ctx, x, T, wts, cache, 0, idx, gw, out)
                ri, rw, ro = ref.forward(x)
                torch.cuda.synchronize()
                assert np.array_equal(idx.cpu().numpy(), ri.cpu().numpy()), (T, s_)
                assert torch.equal(out.view(torch.int32), ro.view(torch.int32)), (T, s_)
                abi.moe_cache_release(cache, 0)
        assert abi.moe_cache_stats_get(cache)["bytes_copied"] > 0
    finally:
        if ctx:
            abi.moe_ctx_destroy(ctx)
        if cache:
            abi.moe_cache_destroy(cache)
        if ref:
            ref.close()
        abi.moe_host_free_pinned(host)
