#!/usr/bin/env python3
"""Throughput of one quantised MoE layer on one MI355X.

Default workload (the decode headline): a GLM-shaped MoE layer with hidden
6144, 256 routed experts + 1 shared expert, FFN 2048 SwiGLU, int4 weights in
groups of 32 with fp16 scales, top-8 sigmoid router with selection bias
N(0, 0.01), routed scale 2.5; batch 1 token per step with fresh N(0,1)
activations every step.  A step is one moe_layer_forward: router logits and
token quantisation, top-k (beside it the shared expert's gate/up + SwiGLU),
routed gate/up + SwiGLU, then requantisation, down projections and combine.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Prints one JSON line.  `value` is layer tokens/s with all inputs resident in
HBM; `roofline` covers the dominant kernel (the routed gate/up projection), its
duration the average of the kernel's own dispatch timestamps (HIP events)
over a pass of the same K steps run back to back; `cpu_baseline` is the plain C oracle on a
bounded sample of the same workload, on this host.
"""
import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s (decode bs1, prefill 4096) + % HBM BW / % int8 MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, datasheet
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, datasheet

H, F, E, K_TOP, G = 6144, 2048, 256, 8, 32
R_SCALE = 2.5


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gu_section_bytes(H_, F_, g):
    return F_ * H_ + (F_ // 8) * (H_ // g) * 32          # nibbles + fp16 scales of 2F rows


def dn_section_bytes(H_, F_, g):
    return H_ * F_ // 2 + (H_ // 16) * (F_ // g) * 32


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_glm_bs1_hbm_traffic.md")


def measured_traffic():
    """HBM bytes per gate/up launch from the committed rocprofv3 counter
    summary, or None when a kernel source listed there has changed since."""
    import hashlib
    try:
        text = open(TRAFFIC_RECORD).read()
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        for path, digest in rec["sources_sha256"].items():
            with open(os.path.join(ROOT, path), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != digest:
                    return None
        return rec["traffic_bytes_per_launch"]
    except (OSError, IndexError, KeyError, ValueError):
        return None


def build_layer(args):
    from quantized_expert_ffn_topk_amd import abi, synth
    from quantized_expert_ffn_topk_amd.layer import Layer, make_desc
    t0 = time.time()
    D = args.distinct
    distinct = [synth.expert_int4(0, e, H, F, G) for e in range(D)]
    shared = synth.expert_int4(0, -1, H, F, G)
    Wr, b = synth.router_weights(0, E, H)
    desc = make_desc(H, F, E, K_TOP, 1, G, R_SCALE)
    lay = Layer(desc, Wr, b, distinct, shared, [e % D for e in range(E)], max_tokens=1)
    log("layer built in %.1f s (%d distinct synthetic experts behind %d device blobs)" % (
        time.time() - t0, D, E))
    return lay, dict(distinct=distinct, shared=shared, Wr=Wr, b=b)


def run_decode(args, lay):
    import torch
    from quantized_expert_ffn_topk_amd import abi, synth
    n_x = args.warmup + args.steps + args.profile_steps
    xs_host = synth.activations(1, n_x, H)
    xs = lay.x_tensor(xs_host)
    idx = torch.empty((1, K_TOP), dtype=torch.int32, device=lay.dev)
    w = torch.empty((1, K_TOP), dtype=torch.float32, device=lay.dev)
    out = torch.empty((1, H), dtype=torch.float32, device=lay.dev)
    stream = torch.cuda.Stream()
    outs = (idx, w, out)

    def step(i):
        lay.forward(xs[i:i + 1], stream=stream, outs=outs)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()

    base = args.warmup
    res = {}
    # eager launches
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(base + i)
    stream.synchronize()
    torch.cuda.synchronize()
    res["eager_s"] = time.perf_counter() - t0
    # the same K steps again with every kernel stamped by start and stop
    # events from its own dispatch (hipExtLaunchKernelGGL) on the launch
    # stream; the library reads them only after the loop, so the steps run
    # back to back and the per-kernel durations are those of the pipeline
    abi.moe_ctx_profile(lay.ctx, True)
    abi.moe_ctx_profile_read(lay.ctx)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(base + i)
    stream.synchronize()
    torch.cuda.synchronize()
    res["profiled_s"] = time.perf_counter() - t0
    prof = abi.moe_ctx_profile_read(lay.ctx)
    abi.moe_ctx_profile(lay.ctx, False)
    res["kernels_us"] = {k: 1e3 * v[0] / v[1] for k, v in prof.items() if v[1]}
    # the same steps captured once as a HIP graph and replayed
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(args.steps):
                step(base + i)
        g.replay()                       # first replay (untimed)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
        stream.synchronize()
        torch.cuda.synchronize()
        res["graph_s"] = time.perf_counter() - t0
        res["graph_event_s"] = ev0.elapsed_time(ev1) / 1e3
        del g
    # spread of single steps: events on the launch stream around each eager step
    pbase = args.warmup + args.steps
    n_sp = args.profile_steps
    if n_sp >= 10:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_sp)]
        for i in range(n_sp):
            evs[i][0].record(stream)
            step(pbase + i)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        res["step_us"] = percentiles([1e3 * a.elapsed_time(b) for a, b in evs])
    return res


def percentiles(v):
    """p10, median and p90 of a list of durations."""
    v = np.sort(np.asarray(v, dtype=np.float64))
    return {"p10": float(np.percentile(v, 10)), "p50": float(np.percentile(v, 50)),
            "p90": float(np.percentile(v, 90)), "n": int(v.size)}


def run_small_batches(args, lay):
    """Decode steps of 2, 4, 8 and 16 tokens through a second context on the
    same device blobs: tokens/s and time per step (eager launches)."""
    import torch
    from quantized_expert_ffn_topk_amd import abi, synth
    ctx = abi.moe_ctx_create(0, lay.desc, 16)
    stream = torch.cuda.Stream()
    sh = abi.stream_handle(stream)
    res = {}
    for T in (2, 4, 8, 16):
        n = 200
        xs = lay.x_tensor(synth.activations(20 + T, T * (n + 10), H))
        idx = torch.empty((T, K_TOP), dtype=torch.int32, device=lay.dev)
        w = torch.empty((T, K_TOP), dtype=torch.float32, device=lay.dev)
        out = torch.empty((T, H), dtype=torch.float32, device=lay.dev)

        def call(i):
            abi.moe_layer_forward(ctx, xs[i * T:(i + 1) * T], T, lay.weights, None, 0, idx, w,
                                  out, sh)

        for i in range(10):
            call(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            call(i)
        stream.synchronize()
        dt = (time.perf_counter() - t0) / n
        res[str(T)] = {"tokens_per_s": T / dt, "us_per_step": 1e6 * dt}
    abi.moe_ctx_destroy(ctx)
    return res


def run_prefill(args, lay):
    """4096-token prefill through a second context on the same device blobs,
    with the Zipf(1.1)-skewed selection bias."""
    import torch
    from quantized_expert_ffn_topk_amd import abi, synth
    T = args.prefill_tokens
    ctx = abi.moe_ctx_create(0, lay.desc, T)
    bz = torch.from_numpy(synth.zipf_bias(0, E)).to(lay.dev)
    wts = abi.moe_layer_weights(lay.Wr.data_ptr(), bz.data_ptr(), lay.ptrs.data_ptr(),
                                lay.shared_blob.data_ptr())
    xs = [lay.x_tensor(synth.activations(10 + i, T, H)) for i in range(2)]
    idx = torch.empty((T, K_TOP), dtype=torch.int32, device=lay.dev)
    w = torch.empty((T, K_TOP), dtype=torch.float32, device=lay.dev)
    out = torch.empty((T, H), dtype=torch.float32, device=lay.dev)
    stream = torch.cuda.Stream()
    sh = abi.stream_handle(stream)

    def call(i):
        abi.moe_layer_forward(ctx, xs[i % 2], T, wts, None, 0, idx, w, out, sh)

    for i in range(2):
        call(i)
    torch.cuda.synchronize()
    n = args.prefill_calls
    t0 = time.perf_counter()
    for i in range(n):
        call(i)
    stream.synchronize()
    dt = (time.perf_counter() - t0) / n
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for i in range(n):
        evs[i][0].record(stream)
        call(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    call_ms = percentiles([a.elapsed_time(b) for a, b in evs])
    abi.moe_ctx_profile(ctx, True)
    abi.moe_ctx_profile_read(ctx)
    for i in range(n):
        call(i)
    torch.cuda.synchronize()
    prof = abi.moe_ctx_profile_read(ctx)
    abi.moe_ctx_profile(ctx, False)
    loads = np.bincount(idx.cpu().numpy().ravel(), minlength=E)
    abi.moe_ctx_destroy(ctx)
    kus = {k: 1e3 * v[0] / v[1] for k, v in prof.items() if v[1]}
    rows = T * (K_TOP + 1)
    ops = 2.0 * rows * (2 * F * H + H * F)                 # int8 MFMA operations (2 per MAC)
    gemm_us = kus.get("gateup", 0.0) + kus.get("down", 0.0)
    sorted_loads = np.sort(loads)[::-1]
    return {
        "workload": "same layer, prefill of %d tokens, selection bias skewing loads like "
                    "Zipf(1.1)" % T,
        "tokens_per_s": T / dt,
        "ms_per_call": 1e3 * dt,
        "ms_per_call_events": call_ms,
        "int8_mfma": {"ops_per_call": ops, "gemm_us": gemm_us,
                      "achieved_TOPS": ops / (gemm_us * 1e-6) / 1e12,
                      "peak_TOPS": INT8_PEAK_TOPS,
                      "frac": ops / (gemm_us * 1e-6) / 1e12 / INT8_PEAK_TOPS},
        "kernels_us": {k: round(v, 2) for k, v in kus.items()},
        "expert_loads": {"max": int(loads.max()), "empty": int((loads == 0).sum()),
                         "top8_share": float(sorted_loads[:8].sum() / loads.sum()),
                         "top32_share": float(sorted_loads[:32].sum() / loads.sum())},
    }


def run_mx(args):
    """MXFP4 wide layer: hidden 7168, 384 routed + 1 shared, F 2048, top-8,
    64 tokens per call, routed scale 1.0, uniform routing bias."""
    import torch
    from quantized_expert_ffn_topk_amd import abi, synth
    from quantized_expert_ffn_topk_amd.layer import Layer, make_desc
    Hm, Fm, Em, Tm = 7168, 2048, 384, 64
    t0 = time.time()
    D = args.mx_distinct
    distinct = [synth.expert_mxfp4(0, e, Hm, Fm) for e in range(D)]
    shared = synth.expert_mxfp4(0, -1, Hm, Fm)
    Wr, _ = synth.router_weights(0, Em, Hm)
    b = synth.uniform_bias(0, Em)
    desc = make_desc(Hm, Fm, Em, K_TOP, 1, 32, 1.0, abi.WFMT_MXFP4)
    lay = Layer(desc, Wr, b, distinct, shared, [e % D for e in range(Em)], max_tokens=Tm)
    log("mxfp4 layer built in %.1f s" % (time.time() - t0))
    xs = [lay.x_tensor(synth.activations(20 + i, Tm, Hm)) for i in range(4)]
    idx, w, out = lay._outs(Tm)
    stream = torch.cuda.Stream()
    sh = abi.stream_handle(stream)

    def call(i):
        abi.moe_layer_forward(lay.ctx, xs[i % 4], Tm, lay.weights, None, 0, idx, w, out, sh)

    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    n = args.mx_calls
    uniq = []
    t0 = time.perf_counter()
    for i in range(n):
        call(i)
    stream.synchronize()
    dt = (time.perf_counter() - t0) / n
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for i in range(n):
        evs[i][0].record(stream)
        call(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    call_ms = percentiles([a.elapsed_time(b) for a, b in evs])
    for i in range(4):                     # experts touched per input
        call(i)
        torch.cuda.synchronize()
        uniq.append(len(np.unique(idx.cpu().numpy())))
    abi.moe_ctx_profile(lay.ctx, True)
    abi.moe_ctx_profile_read(lay.ctx)
    for i in range(n):
        call(i)
    torch.cuda.synchronize()
    prof = abi.moe_ctx_profile_read(lay.ctx)
    abi.moe_ctx_profile(lay.ctx, False)
    kus = {k: 1e3 * v[0] / v[1] for k, v in prof.items() if v[1]}
    blob = abi.moe_blob_bytes(desc)
    touched = float(np.mean(uniq)) + 1.0
    layer_bytes = touched * blob + Em * Hm * 4
    ffn_us = kus.get("gateup", 0.0) + kus.get("down", 0.0)
    lay.close()
    return {
        "workload": "MXFP4 wide layer: hidden 7168, 384 routed + 1 shared experts, FFN 2048, "
                    "top-8, E2M1 + E8M0 per 32, bf16 activations, 64 tokens per call, routed "
                    "scale 1.0, bias U(-0.01, 0.01)",
        "tokens_per_s": Tm / dt,
        "ms_per_call": 1e3 * dt,
        "ms_per_call_events": call_ms,
        "experts_touched_per_call": touched,
        "hbm": {"bytes_per_call": layer_bytes,
                "layer_GBs": layer_bytes / dt / 1e9,
                "layer_frac": layer_bytes / dt / 1e9 / HBM_PEAK_GBS,
                "expert_ffn_GBs": touched * blob / (ffn_us * 1e-6) / 1e9 if ffn_us else None},
        "kernels_us": {k: round(v, 2) for k, v in kus.items()},
    }


def run_stream(args, lay, W):
    """Expert streaming: 16 GLM-shaped layers whose 4096 routed experts live in
    pinned host memory behind a 24 GiB HBM cache (global LRU), decode batch 1,
    Zipf(1.1) routing with 70 % layer-to-layer correlation imposed through the
    selection bias, successor-set lookahead prefetch of the next layer."""
    import ctypes as C
    import torch
    from quantized_expert_ffn_topk_amd import abi, synth
    L, steps = 16, args.stream_steps
    blob = abi.moe_blob_bytes(lay.desc)
    n_phys = args.stream_phys
    # the 4096 keys alias n_phys pinned blobs: the copy traffic is the same
    host = abi.moe_host_alloc_pinned(n_phys * blob)
    try:
        base = np.ctypeslib.as_array(C.cast(host, C.POINTER(C.c_uint8)), shape=(n_phys * blob,))
        for i in range(n_phys):
            base[i * blob:(i + 1) * blob] = lay.blobs[i % len(lay.blobs)].cpu().numpy()
        ptrs = (C.c_void_p * (L * E))(*[host + ((l * E + e) % n_phys) * blob
                                         for l in range(L) for e in range(E)])
        cap = 24 << 30
        cache = abi.moe_cache_create(abi.moe_cache_desc(0, L, E, blob, cap, C.addressof(ptrs),
                                                        abi.CACHE_GLOBAL_LRU, abi.CACHE_BACKEND_HIP))
        demand, predict = synth.zipf_trace(3, L, E, K_TOP, steps)
        bias = torch.from_numpy(np.stack([[synth.forcing_bias(E, demand[t, l]) for l in range(L)]
                                          for t in range(steps)])).to(lay.dev)
        ctx = abi.moe_ctx_create(0, lay.desc, 1)
        xs = lay.x_tensor(synth.activations(30, steps * L, H))
        idx, w, out = lay._outs(1)
        stream = torch.cuda.Stream()
        sh = abi.stream_handle(stream)

        def layer_call(t, l):
            wts = abi.moe_layer_weights(lay.Wr.data_ptr(), bias[t, l].data_ptr(), None,
                                        lay.shared_blob.data_ptr())
            abi.moe_layer_forward(ctx, xs[t * L + l:t * L + l + 1], 1, wts, cache, l, idx, w, out, sh)
            if l + 1 < L:
                abi.moe_cache_stage(cache, l + 1, predict[t, l], abi.STAGE_PREFETCH, sh)
            abi.moe_cache_release(cache, l, sh)

        warm = min(8, steps // 4)
        for t in range(warm):
            for l in range(L):
                layer_call(t, l)
        torch.cuda.synchronize()
        abi.moe_cache_reset_stats(cache)
        t0 = time.perf_counter()
        for t in range(warm, steps):
            for l in range(L):
                layer_call(t, l)
        stream.synchronize()
        dt = time.perf_counter() - t0
        st = abi.moe_cache_stats_get(cache)
        abi.moe_ctx_destroy(ctx)
        abi.moe_cache_destroy(cache)
    finally:
        abi.moe_host_free_pinned(host)
    # pinned host -> device ceiling on this machine, same blob size
    src = torch.empty(blob * 32, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(blob * 32, dtype=torch.uint8, device=lay.dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(3):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    ceil_gbs = 3 * blob * 32 / (time.perf_counter() - t1) / 1e9
    n = steps - warm
    dem = st["demand_hits"] + st["demand_misses"]
    return {
        "workload": "expert streaming: 16 GLM-shaped layers, 4096 routed experts of %d B in "
                    "pinned host memory (keys aliased onto %d physical blobs), 24 GiB HBM LRU "
                    "pool (%d slots), decode batch 1, Zipf(1.1) routing with 0.7 layer-to-layer "
                    "correlation, lookahead prefetch of the successor set" % (blob, n_phys,
                                                                               st["n_slots"]),
        "tokens_per_s": n / dt,
        "ms_per_token": 1e3 * dt / n,
        "h2d_GBs": st["bytes_copied"] / dt / 1e9,
        "h2d_pinned_ceiling_GBs": ceil_gbs,
        "demand_hit_rate": st["demand_hits"] / dem if dem else None,
        "prefetch_precision": (st["prefetch_used"] / st["prefetch_issued"]
                               if st["prefetch_issued"] else None),
        "misses_per_token": st["demand_misses"] / n,
        "stats": st,
    }


def cpu_baseline(args, lay, W):
    """The plain C oracle (single thread) on a bounded sample of decode steps."""
    import oracle
    from quantized_expert_ffn_topk_amd import synth
    oracle.lib()
    xs = synth.activations(2, args.cpu_steps_max, H)
    emap = [e % args.distinct for e in range(E)]
    t0 = time.perf_counter()
    n = 0
    while n < args.cpu_steps_max:
        oracle.layer(xs[n:n + 1], W["Wr"], W["b"], W["distinct"], W["shared"], K_TOP, R_SCALE, G,
                     expert_map=emap)
        n += 1
        if time.perf_counter() - t0 > args.cpu_seconds and n >= 2:
            break
    dt = time.perf_counter() - t0
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%d decode steps (batch 1) of the same layer, full 6144-wide output, "
                      "single-threaded C (gcc -O2) on %s; host has %d logical CPUs" % (
                          n, cpu, os.cpu_count() or 0)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--profile-steps", type=int, default=200,
                    help="eager steps timed one by one for the p10/p50/p90 spread")
    ap.add_argument("--distinct", type=int, default=8,
                    help="distinct synthetic experts copied into the 256 device blobs")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-steps-max", type=int, default=40)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-small-batches", action="store_true",
                    help="skip the 2/4/8/16-token decode lines")
    ap.add_argument("--prefill-tokens", type=int, default=4096)
    ap.add_argument("--prefill-calls", type=int, default=5)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (HBM counter "
                         "calibration under rocprofv3 --pmc)")
    ap.add_argument("--no-mx", action="store_true")
    ap.add_argument("--no-stream", action="store_true")
    ap.add_argument("--stream-steps", type=int, default=96)
    ap.add_argument("--stream-phys", type=int, default=48)
    ap.add_argument("--mx-calls", type=int, default=10)
    ap.add_argument("--mx-distinct", type=int, default=4)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    lay, W = build_layer(args)
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=lay.dev)
        b = torch.empty(n, dtype=torch.uint8, device=lay.dev)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log("calibration copy of %d MiB done" % args.calib_copy_mib)
        del a, b
    res = run_decode(args, lay)
    K = args.steps
    best = min(res["eager_s"], res.get("graph_s", 1e30))
    ms_per_step = 1e3 * best / K
    # algorithmic bytes per launch: weights + scales of the experts it runs,
    # the int8 token codes once, the fp32 SwiGLU rows (gate/up); the SwiGLU rows
    # read, the per-slot projections and the output written (down)
    gu_bytes = K_TOP * gu_section_bytes(H, F, G) + H + K_TOP * F * 4
    gu_us = res["kernels_us"]["gateup"]
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    S = K_TOP + 1
    dn_bytes = S * dn_section_bytes(H, F, G) + S * F * 4 + S * H * 4 + H * 4
    dn_us = res["kernels_us"]["down"]
    layer_bytes = S * (gu_section_bytes(H, F, G) + dn_section_bytes(H, F, G)) + E * H * 4
    line = {
        "metric": METRIC,
        "value": K / best,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {
            "workload": "GLM-shaped MoE layer decode, batch 1: hidden 6144, 256 routed + 1 shared "
                        "experts, FFN 2048 SwiGLU, int4 group-32 fp16 scales, int8 activations, "
                        "top-8 sigmoid router with bias N(0,0.01), routed scale 2.5, fresh "
                        "N(0,1) tokens each step",
            "global_batch": 1,
            "timing": "graph replay" if best == res.get("graph_s") else "eager launches",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "gateup_bs1_kernel (gate/up projections + SwiGLU of the 8 routed experts)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(),
            "bytes_per_launch": gu_bytes,
            "avg_us": gu_us,
        },
        "gemv_hbm": {
            "down_achieved_GBs": dn_bytes / (dn_us * 1e-6) / 1e9,
            "down_bytes_per_launch": dn_bytes,
            # every weight byte of the step (9 experts + router) over the step time
            "layer_bytes_per_step": layer_bytes,
            "layer_GBs": layer_bytes / (ms_per_step * 1e-3) / 1e9,
            "layer_frac": layer_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        },
        "kernels_us": {k: round(v, 3) for k, v in res["kernels_us"].items()},
        "step_us_eager": res.get("step_us"),
        "eager_tokens_per_s": K / res["eager_s"],
        "profiled_eager_tokens_per_s": K / res["profiled_s"],
        "graph_tokens_per_s": (K / res["graph_s"]) if "graph_s" in res else None,
    }
    if not args.no_small_batches:
        line["decode_small_batches"] = run_small_batches(args, lay)
    if not args.no_prefill:
        line["prefill"] = run_prefill(args, lay)
    if not args.no_stream:
        line["streaming"] = run_stream(args, lay, W)
    if not args.no_mx:
        line["mxfp4"] = run_mx(args)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args, lay, W)
    else:
        line["cpu_baseline"] = None
    line["host"] = platform.node()
    print(json.dumps(line), flush=True)
    lay.close()


if __name__ == "__main__":
    main()
