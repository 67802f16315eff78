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

    def __init__(self, n_slots, policy=abi.CACHE_GLOBAL_LRU):
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
                          self.shared[l], max_tokens=1) for l in range(L_)]
        self.ctx = abi.moe_ctx_create(0, self.desc, 1)
        self.bias = torch.zeros(E, dtype=torch.float32, device="cuda")
        self.wts = [abi.moe_layer_weights(self.ref[l].Wr.data_ptr(), self.bias.data_ptr(), None,
                                          self.ref[l].shared_blob.data_ptr()) for l in range(L_)]

    def close(self):
        abi.moe_ctx_destroy(self.ctx)
        abi.moe_cache_destroy(self.cache)
        for r in self.ref:
            r.close()
        abi.moe_host_free_pinned(self.host)


def _run(stk, demand, predict, steps):
    """The streaming loop: layer l runs through the cache (DEMAND inside the
    forward), then the guess for the next layer is prefetched and layer l is
    released; every output is checked against the resident layer."""
    used = np.empty_like(demand[:steps])
    idx = torch.empty((1, K), dtype=torch.int32, device="cuda")
    gw = torch.empty((1, K), dtype=torch.float32, device="cuda")
    out = torch.empty((1, H), dtype=torch.float32, device="cuda")
    for t in range(steps):
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
                abi.moe_cache_stage(stk.cache, nl, predict[t, l], abi.STAGE_PREFETCH)
            abi.moe_cache_release(stk.cache, l)
    torch.cuda.synchronize()
    return used


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
