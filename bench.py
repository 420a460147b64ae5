#!/usr/bin/env python3
"""Benchmark of the int4 routed-expert MoE block on one MI355X.

Default workload: the 80B-shaped batched layer stack (48 layers, hidden 2048,
512 experts, top-10, expert and shared intermediate 512, int4 affine group 64,
64 tokens per step, Zipf(1.3) router bias), all experts resident in HBM with
distinct seeded weights per layer.  One step = the whole stack (router, top-k,
bucketing, gate/up+SwiGLU, down, combine, residual epilogue) for 64 tokens,
replayed as one captured HIP graph.

Prints one JSON line: tokens/s, int4-expert-byte GB/s, the dominant kernel's
roofline (HIP events around it, inside a replay of the same graph) and the
fp64 oracle's throughput on the host cores for a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="bat80", choices=["bat80", "dec80", "dec35", "pool80", "dec80i8", "bat80i8", "gdn80"])
    ap.add_argument("--layers", type=int, default=0, help="override the number of layers (0 = workload's)")
    ap.add_argument("--path", type=int, default=0, help="0 auto, 1 GEMV family, 2 grouped family")
    ap.add_argument("--eager", action="store_true", help="launch kernels one by one instead of a HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--pregate", type=int, default=0,
                    help="pool80: prefetch this many of the next layer's predicted experts per layer (0 = none)")
    ap.add_argument("--pool-copy", default="kernel", choices=["kernel", "engine"],
                    help="pool80 host driver: copy misses with the copy kernel (mapped host reads) or the copy engine")
    ap.add_argument("--pool-driver", default="device", choices=["device", "host"],
                    help="pool80: the GPU-resident pool, one captured graph per token (device), or the host "
                         "policy with a per-layer index read-back (host)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (scale reference for HBM byte counters)")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="only measure plain streaming reads (read sizes x workgroup counts): the practical HBM "
                         "read ceiling the FFN kernels are compared with")
    return ap.parse_args()


COPY_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gateup_bat80.txt")
GROUPED_SRC = os.path.join(ROOT, "int4_routed_expert_router_amd", "csrc", "moe_ffn_grouped.hip")
GDN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gdn_step_gdn80.txt")
GDN_SRC = os.path.join(ROOT, "int4_routed_expert_router_amd", "csrc", "gdn.hip")


def copy_calibration():
    """A plain device-to-device copy of COPY_BYTES, three times: under
    rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE per dispatch give the factor
    that turns those counters into bytes."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_dispatch": COPY_BYTES, "dispatches": 3}))


def read_ceiling():
    """Plain streaming reads of windows of a 4 GiB buffer (so each read comes
    from HBM, not the 256 MB Infinity Cache: consecutive launches read
    different windows, as the 48 layers of a stack do), for read sizes of one
    FFN launch (16 and 50 MB) and 1 GiB, and 256 to 2048 workgroups of 512
    threads.  HIP events on the launch stream around every launch; one JSON
    line per (size, workgroups) with the average rate."""
    import ctypes as C
    import torch
    from int4_routed_expert_router_amd._lib import check, lib
    buf_bytes = 4 << 30
    buf = torch.empty(buf_bytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(65536, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    base = buf.data_ptr()
    for size in (16 << 20, 50 << 20, 1 << 30):
        n_win = buf_bytes // size
        for wgs in (256, 512, 1024, 2048):
            reps = min(48, 4 * n_win)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            with torch.cuda.stream(stream):
                for w in range(3):   # warm-up launches
                    check(lib().moe_read_probe(C.c_void_p(base + (w % n_win) * size), size, wgs,
                                               C.c_void_p(sink.data_ptr()), C.c_void_p(stream.cuda_stream)))
                for i in range(reps):
                    ev[i][0].record(stream)
                    check(lib().moe_read_probe(C.c_void_p(base + ((i + 3) % n_win) * size), size, wgs,
                                               C.c_void_p(sink.data_ptr()), C.c_void_p(stream.cuda_stream)))
                    ev[i][1].record(stream)
            torch.cuda.synchronize()
            us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
            print(json.dumps({"read_bytes": size, "workgroups": wgs, "launches": reps, "avg_us": round(us, 2),
                              "GBps": round(size / (us * 1e-6) / 1e9, 1),
                              "frac_of_8TBps": round(size / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}), flush=True)

    def events_avg(addrs, size, wgs):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in addrs]
        with torch.cuda.stream(stream):
            for i, a in enumerate(addrs):
                ev[i][0].record(stream)
                check(lib().moe_read_probe(C.c_void_p(a), size, wgs, C.c_void_p(sink.data_ptr()),
                                           C.c_void_p(stream.cuda_stream)))
                ev[i][1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev[3:]])) * 1e3

    # the fixed cost of event timing itself: 16 KiB read by one workgroup
    print(json.dumps({"case": "16 KiB by one workgroup (event timing floor)",
                      "avg_us": round(events_avg([base] * 40, 16384, 1), 2)}), flush=True)
    # fresh pages or not: windows rotating over smaller spans, and one window re-read
    for size in (16 << 20, 50 << 20):
        for span in (1 << 30, 512 << 20):
            n = span // size
            print(json.dumps({"case": "rotating windows", "read_bytes": size, "span_bytes": span,
                              "avg_us": round(events_avg([base + (i % n) * size for i in range(40)], size, 256), 2)}),
                  flush=True)
        print(json.dumps({"case": "one window re-read (Infinity Cache)", "read_bytes": size,
                          "avg_us": round(events_avg([base] * 40, size, 256), 2)}), flush=True)


def measured_traffic(path=TRAFFIC_FILE, src=GROUPED_SRC):
    """HBM bytes per launch of a kernel from its committed counter summary, or
    None when the kernel source changed since the counters were taken."""
    import hashlib
    try:
        text = open(path).read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    src_hash = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if vals.get("kernel_source_sha256") != src_hash:
        return None
    try:
        fetch = float(vals["fetch_kib_per_launch"]) * 1024 * float(vals["copy_fetch_bytes_per_kib"]) / 1024
        write = float(vals["write_kib_per_launch"]) * 1024 * float(vals["copy_write_bytes_per_kib"]) / 1024
    except (KeyError, ValueError):
        return None
    return fetch + write


class Stack:
    """Device-resident synthetic layer stack (weights generated on the GPU)."""

    def __init__(self, wl, n_layers, path=0):
        import torch
        import synth
        from int4_routed_expert_router_amd import api
        self.wl, self.L = wl, n_layers
        self.desc = api.Desc(wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter, wl.group, wl.act_dtype,
                             path, wl.bits)
        self.stride = api.blob_bytes(wl.hidden, wl.inter, wl.group, wl.bits)
        self.sstride = api.blob_bytes(wl.hidden, wl.shared_inter, wl.group, wl.bits)
        E = wl.n_experts
        self.slab = torch.empty(n_layers * E * self.stride, dtype=torch.uint8, device="cuda")
        self.shared = torch.empty(n_layers * self.sstride, dtype=torch.uint8, device="cuda")
        self.layers = []
        for l in range(n_layers):
            ex = self.slab[l * E * self.stride:(l + 1) * E * self.stride]
            sh = self.shared[l * self.sstride:(l + 1) * self.sstride]
            api.synth_fill_experts(wl.weight_seed, l, 0, E, wl.hidden, wl.inter, wl.group, wl.scale_lo, wl.scale_hi,
                                   ex, self.stride, bits=wl.bits)
            api.synth_fill_experts(wl.weight_seed, l, E, 1, wl.hidden, wl.shared_inter, wl.group, wl.scale_lo,
                                   wl.scale_hi, sh, self.sstride, bits=wl.bits)
            wr = torch.from_numpy(synth.router_weights(wl, l).view(np.int16).copy()).cuda()
            b = synth.router_bias(wl, l)
            bt = None if b is None else torch.from_numpy(b).cuda()
            self.layers.append(api.Layer(wr, bt, ex, self.stride, None, sh))
        T = wl.tokens
        self.T = T
        x_bits = synth.tokens(wl)
        self.x0 = torch.from_numpy(x_bits.view(np.int16).copy()).cuda()
        xf = (x_bits.astype(np.uint32) << 16).view(np.float32) if wl.act_dtype == "bf16" else \
            x_bits.view(np.float16).astype(np.float32)
        self.r0 = torch.from_numpy(xf.copy()).cuda()
        self.r = self.r0.clone()
        self.x_buf = torch.empty_like(self.x0)
        self.ws = api.workspace(self.desc, T)
        self.idx_all = torch.empty(n_layers, T, wl.top_k, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()

    def run_eager(self, stream=None):
        from int4_routed_expert_router_amd import api
        self.r.copy_(self.r0)
        api.stack_forward(self.desc, self.layers, self.x0, self.r, self.x_buf, self.ws, idx_all=self.idx_all,
                          stream=stream)

    def capture(self, stream):
        from int4_routed_expert_router_amd import api
        return api.StackGraph(self.desc, self.layers, self.x0, self.r, self.x_buf, self.ws, stream,
                              idx_all=self.idx_all)

    def active_experts(self):
        idx = self.idx_all.cpu().numpy()
        return [len(np.unique(idx[l])) for l in range(self.L)]


def kernel_events(n):
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n)] for _ in range(2)]
    for e in ev[0] + ev[1]:
        e.record()          # torch creates the underlying hipEvent on first record
    torch.cuda.synchronize()
    return ev[0], ev[1]


def set_timer(begin, end, kind):
    import ctypes as C
    from int4_routed_expert_router_amd._lib import check, lib
    arr_b = (C.c_void_p * len(begin))(*[e.cuda_event for e in begin])
    arr_e = (C.c_void_p * len(end))(*[e.cuda_event for e in end])
    check(lib().moe_stack_set_kernel_events(arr_b, arr_e, len(begin), kind))


def clear_timer():
    from int4_routed_expert_router_amd._lib import check, lib
    check(lib().moe_stack_set_kernel_events(None, None, 0, 0))


def cpu_baseline(wl, budget_s):
    """fp64 oracle on a bounded sample: whole layers of the same workload
    (all tokens), as many as fit the budget (at least one).  Each layer's
    inputs (the quantised weights of the experts it selects, router weights
    and bias) are generated before its timer starts; the timed part is the
    oracle itself: routing, dequantisation of the selected experts, SwiGLU
    FFNs and combine."""
    import synth
    from oracle import moe_oracle as mo
    cores = len(os.sched_getaffinity(0))
    x64 = mo.act_bits_to_f64(synth.tokens(wl), wl.act_dtype)
    timed, gen = 0.0, 0.0
    done = 0
    while True:
        l = done
        g0 = time.perf_counter()
        wr = mo.f16_bits_to_f64(synth.router_weights(wl, l))
        b = synth.router_bias(wl, l)
        b64 = None if b is None else b.astype(np.float64)
        # the experts the layer will select (routing is repeated, timed, below)
        touched = sorted(set(mo.route(x64, wr, b64, wl.top_k)[0].ravel().tolist()))
        raw = {e: synth.expert_raw(wl, l, e) for e in touched}
        raw_shared = synth.expert_raw(wl, l, 0, shared=True)
        gen += time.perf_counter() - g0

        def expert(e, raw=raw):
            r = raw[e]
            return mo.ExpertWeights.from_quant(r["gate"], r["up"], r["down"], wl.group, wl.bits)

        t0 = time.perf_counter()
        shared = mo.ExpertWeights.from_quant(raw_shared["gate"], raw_shared["up"], raw_shared["down"], wl.group,
                                             wl.bits)
        mo.layer_forward(x64, wr, b64, expert, shared, wl.top_k)
        timed += time.perf_counter() - t0
        done += 1
        if timed >= budget_s or done >= wl.layers:
            break
    per_layer = timed / done
    tok_s = wl.tokens / (per_layer * wl.layers)
    return dict(value=tok_s, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{done} whole layer(s) x {wl.tokens} tokens of the same workload: {timed:.1f} s of oracle "
                       f"time (routing, dequantisation of the selected experts, FFNs, combine), scaled to the "
                       f"{wl.layers}-layer stack; input generation ({gen:.1f} s) outside the timer")


def run_pool(args):
    """Slot-pool streaming (pool80): all 48 x 512 expert blobs in pinned host
    memory, 128 HBM slots per layer, batch-1 decode for the workload's steps
    with the router bias re-drawn every drift period.  Each token is one call
    of the native driver (moe_pool_decode_step): per layer, route (and, with
    pre-gating, the next layer's router on this layer's input), read the
    indices back, acquire (misses copied on a side stream), prefetch the
    predicted experts of the next layer (their copies overlap this layer's
    FFN and the next routing), expert FFN from the slots, residual epilogue,
    release.  Reports tokens/s, hit rate and the bytes copied host to
    device."""
    import torch
    import synth
    from int4_routed_expert_router_amd import api
    wl = synth.POOL80
    L = args.layers or wl.layers
    E, H, K, S = wl.n_experts, wl.hidden, wl.top_k, wl.slots_per_layer
    stride = api.blob_bytes(H, wl.inter, wl.group)
    sstride = api.blob_bytes(H, wl.shared_inter, wl.group)
    steps = args.steps if args.steps != 20 else wl.steps
    print(f"[bench] pool80: pinning {L * E * stride / 1e9:.1f} GB of host blobs ...", file=sys.stderr, flush=True)
    t0 = time.time()
    host = torch.empty(L * E * stride, dtype=torch.uint8, pin_memory=True)
    stage = torch.empty(E * stride, dtype=torch.uint8, device="cuda")
    shared = torch.empty(L * sstride, dtype=torch.uint8, device="cuda")
    routers, biases = [], []
    epochs = (steps + wl.drift_period - 1) // wl.drift_period
    for l in range(L):
        api.synth_fill_experts(wl.weight_seed, l, 0, E, H, wl.inter, wl.group, wl.scale_lo, wl.scale_hi, stage,
                               stride)
        api.synth_fill_experts(wl.weight_seed, l, E, 1, H, wl.shared_inter, wl.group, wl.scale_lo, wl.scale_hi,
                               shared[l * sstride:(l + 1) * sstride], sstride)
        host[l * E * stride:(l + 1) * E * stride].copy_(stage)
        routers.append(torch.from_numpy(synth.router_weights(wl, l).view(np.int16).copy()).cuda())
        biases.append([torch.from_numpy(synth.router_bias(wl, l, epoch=ep)).cuda() for ep in range(epochs)])
    del stage
    slab = torch.empty(L * S * stride, dtype=torch.uint8, device="cuda")
    offsets = torch.zeros(L * E, dtype=torch.int64, device="cuda")
    copy_stream = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    device_pool = args.pool_driver == "device"
    if device_pool:
        pool = api.DevPool(L, E, S, wl.drift_period, stride, stride, host, slab, offsets)
    else:
        pool = api.SlotPool(L, E, S, wl.drift_period, stride, stride, host, slab, offsets, copy_stream,
                            dma_copy=args.pool_copy == "engine")
    desc = api.Desc(H, E, K, wl.inter, wl.shared_inter, wl.group, wl.act_dtype, 0)
    ws = api.workspace(desc, 1)
    toks = torch.from_numpy(np.stack([synth.tokens(wl, step=s)[0] for s in range(steps)]).view(np.int16)).cuda()
    x_buf = torch.empty(2, H, dtype=torch.int16, device="cuda")
    r = torch.empty(H, dtype=torch.float32, device="cuda")
    idx_host = torch.empty(2, K, dtype=torch.int32, pin_memory=True)
    pregate = args.pregate
    layers = [[api.Layer(routers[l], biases[l][ep], slab, stride, offsets, shared[l * sstride:]) for l in range(L)]
              for ep in range(epochs)]
    graphs = []
    x0 = torch.empty(1, H, dtype=torch.int16, device="cuda")
    if device_pool:
        # one captured token graph per drift epoch (the router bias differs),
        # captured on and launched from a stream of its own
        compute = torch.cuda.Stream()
        graphs = [api.PoolGraph(desc, layers[ep], pool, x0, r, x_buf, ws, compute) for ep in range(epochs)]
    torch.cuda.synchronize()
    print(f"[bench] pool80 ready in {time.time() - t0:.1f} s; {steps} steps x {L} layers", file=sys.stderr,
          flush=True)
    t_start = time.perf_counter()
    with torch.cuda.stream(compute):
        for s in range(steps):
            x = toks[s:s + 1]
            r.copy_(x.view(torch.bfloat16).float()[0])
            if device_pool:
                x0.copy_(x)
                graphs[s // wl.drift_period].launch(compute)
            else:
                api.pool_decode_step(desc, layers[s // wl.drift_period], pool, s, x, r, x_buf, idx_host, ws,
                                     pregate=pregate, stream=compute)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    st = pool.stats()
    req = st["hits"] + st["misses"]
    out = {"metric": "slot-pool streaming decode tokens/sec (80B-shaped, 25% of experts in HBM)",
           "value": round(steps / elapsed, 2), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
           "ms_per_step": round(1e3 * elapsed / steps, 3), "higher_is_better": True,
           "hit_rate": round(st["hits"] / max(req, 1), 4), "hits": st["hits"], "misses": st["misses"],
           "evictions": st["evictions"], "prefetches": st["prefetches"], "bytes_h2d": st["bytes_h2d"],
           "h2d_GBps": round(st["bytes_h2d"] / elapsed / 1e9, 2),
           "config": {"workload": f"pool80: {L} layers x {E} experts as pinned host blobs of {stride} B, "
                                  f"{S} HBM slots per layer, batch 1, {steps} steps, router bias re-drawn every "
                                  f"{wl.drift_period} steps, router weights x3, "
                                  + ("GPU-resident pool (policy kernel, miss copies by a kernel reading a "
                                     "device miss list), one captured graph per token" if device_pool else
                                     ("host policy, " + (f"pre-gated prefetch of the top {pregate} predictions of "
                                      "the next layer" if pregate else "no prefetch")
                                      + f", copies by the copy {args.pool_copy}"))},
           "data": "synthetic (seeded)"}
    pool.close()
    print(json.dumps(out))


def run_gdn(args):
    """Gated DeltaNet decode step (gdn80): one token for each of 64 sequences
    through 36 DeltaNet layers, every layer's [32 heads][128][128] fp32 state
    per sequence resident in HBM (4.8 GB) and updated in place.  One step =
    36 launches of moe_gdn_step."""
    import math
    import torch
    import synth
    from int4_routed_expert_router_amd import api
    from oracle import deltanet_oracle as dn
    from oracle import moe_oracle as mo
    wl = synth.GDN80
    L = args.layers or wl.layers
    B, Hk, Hv, dk, dv = wl.batch, wl.k_heads, wl.v_heads, wl.head_k_dim, wl.head_v_dim
    qs = 1.0 / math.sqrt(dk)
    print(f"[bench] gdn80: {L} layers x {B} sequences, state {L * B * Hv * dv * dk * 4 / 1e9:.2f} GB",
          file=sys.stderr, flush=True)
    states, ins = [], []
    for l in range(L):
        states.append(torch.from_numpy(synth.gdn_state(wl, l)).cuda())
        q, k, v, g, beta = synth.gdn_inputs(wl, l, 0)
        ins.append([torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()
                    for a in (q, k, v, g, beta)])
    o = torch.empty(B, Hv, dv, dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()

    def step():
        for l in range(L):
            q, k, v, g, beta = ins[l]
            api.gdn_step(q, k, v, g, beta, states[l], o, qs, wl.act_dtype, stream=stream)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        # HIP events on the launch stream around every layer's launch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(L)]
        durs = []
        for _ in range(max(3, min(args.steps, 10))):
            for l in range(L):
                q, k, v, g, beta = ins[l]
                ev[l][0].record(stream)
                api.gdn_step(q, k, v, g, beta, states[l], o, qs, wl.act_dtype, stream=stream)
                ev[l][1].record(stream)
            torch.cuda.synchronize()
            durs += [ev[l][0].elapsed_time(ev[l][1]) for l in range(L)]
    avg_us = float(np.mean(durs)) * 1e3
    tb = measured_traffic(GDN_TRAFFIC_FILE, GDN_SRC)
    state_b = B * Hv * dv * dk * 4
    per_launch = 2 * state_b + 2 * B * Hk * dk * 2 + B * Hv * dv * 2 + B * Hv * 8 + B * Hv * dv * 4
    achieved = per_launch / (avg_us * 1e-6) / 1e9
    ms = 1e3 * elapsed / args.steps
    print(f"[bench] {ms:.3f} ms/step, {B * args.steps / elapsed:.0f} tok/s, launch {avg_us:.2f} us, "
          f"{achieved:.0f} GB/s", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle on whole layers (all 64 sequences), as many as fit the budget
        q, k, v, g, beta = synth.gdn_inputs(wl, 0, 0)
        host = [mo.act_bits_to_f64(a, wl.act_dtype) for a in (q, k, v)] + [g.astype(np.float64), beta.astype(np.float64)]
        st = synth.gdn_state(wl, 0).astype(np.float64)
        t0 = time.perf_counter()
        done = 0
        while True:
            st, _ = dn.gdn_step(st, *host, qs)
            done += 1
            el = time.perf_counter() - t0
            if el >= min(args.cpu_seconds, 10.0) or done >= L:
                break
        cpu = dict(value=round(B / (el / done * L), 2), unit="tokens/s", cores=len(os.sched_getaffinity(0)),
                   kind="oracle", sample=f"{done} layer step(s) x {B} sequences in {el:.1f} s, scaled to {L} layers")
    out = {"metric": "Gated DeltaNet decode step tokens/sec + state HBM GB/s (80B-shaped, 64 sequences)",
           "value": round(B * args.steps / elapsed, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded)",
           "config": {"workload": f"gdn80: {L} Gated DeltaNet layers, {B} sequences, {Hv} value / {Hk} key heads, "
                                  f"head dims {dk}, state fp32 in place, {wl.act_dtype} q/k/v"},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": None if tb is None else round(tb / (avg_us * 1e-6) / 1e9, 1),
                        "kernel": "k_gdn_step", "avg_us": round(avg_us, 2), "bytes_per_launch": int(per_launch),
                        "traffic_bytes_per_launch": None if tb is None else int(tb),
                        "events": "HIP events on the launch stream around each layer's launch"},
           "cpu_baseline": cpu}
    print(json.dumps(out))


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.read_ceiling:
        read_ceiling()
        return
    if args.gpus != 1:
        print(json.dumps({"error": f"--gpus {args.gpus}: this benchmark runs on exactly one GPU; "
                                   "multi-GPU sharding is designed (DESIGN.md) but not built"}))
        sys.exit(2)
    if args.workload == "pool80":
        run_pool(args)
        return
    if args.workload == "gdn80":
        run_gdn(args)
        return
    import torch
    import synth
    from int4_routed_expert_router_amd._lib import MOE_TIME_GATEUP
    wl = synth.WORKLOADS[args.workload]
    L = args.layers or wl.layers
    print(f"[bench] building {L}-layer {wl.name} stack ...", file=sys.stderr, flush=True)
    t0 = time.time()
    st = Stack(wl, L, args.path)
    print(f"[bench] stack ready in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    stream = torch.cuda.Stream()
    graph = None
    with torch.cuda.stream(stream):
        if not args.eager:
            graph = st.capture(stream)

        def step():
            st.r.copy_(st.r0)
            if graph is not None:
                graph.launch(stream)
            else:
                st.run_eager(stream)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
        # per-step spread, outside the timed region: HIP events on the step's
        # stream around each of another K steps
        step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
        for b_ev, e_ev in step_ev:
            b_ev.record(stream)
            step()
            e_ev.record(stream)
        torch.cuda.synchronize()
        step_ms = np.array([b_ev.elapsed_time(e_ev) for b_ev, e_ev in step_ev])
    ms_per_step = 1e3 * elapsed / args.steps
    tokens_s = wl.tokens * args.steps / elapsed
    act = st.active_experts()
    B = st.stride  # routed and shared blobs have the same size in these workloads
    wname = f"int{wl.bits}"
    expert_bytes = sum((a + 1) * B for a in act)
    expert_gbs = expert_bytes / (ms_per_step * 1e-3) / 1e9
    grouped = args.path == 2 or (args.path == 0 and wl.tokens * wl.top_k > 32)
    print(f"[bench] {ms_per_step:.3f} ms/step, {tokens_s:.0f} tok/s, {wname} {expert_gbs:.0f} GB/s, "
          f"active experts/layer mean {np.mean(act):.1f}", file=sys.stderr, flush=True)

    roof = None
    kernel_us = {}
    kernel_roof = None
    if not args.no_kernel_timing:
        # HIP events around each layer's kernel of one kind, recorded on the
        # stream that launches it, over eager (launch-by-launch) replays of the
        # same steps; event nodes inside a captured graph perturb the replay.
        from int4_routed_expert_router_amd._lib import MOE_TIME_DOWN, MOE_TIME_ROUTER
        reps = max(3, min(args.steps, 10))
        for kind, name in ((MOE_TIME_GATEUP, "gateup"), (MOE_TIME_DOWN, "down"), (MOE_TIME_ROUTER, "router")):
            begin, end = kernel_events(L)
            durs = []
            with torch.cuda.stream(stream):
                for _ in range(reps):
                    set_timer(begin, end, kind)
                    st.run_eager(stream)
                    clear_timer()
                    torch.cuda.synchronize()
                    durs.append([begin[l].elapsed_time(end[l]) for l in range(L)])
            kernel_us[name] = float(np.mean(durs)) * 1e3
        avg_us = kernel_us["gateup"]
        # gate and up values (2 I H of bits/8 bytes) plus their fp16 scale and bias
        gu_bytes = (st.desc.inter * st.desc.hidden * wl.bits // 4
                    + 8 * st.desc.inter * st.desc.hidden // st.desc.group_size)
        per_launch = float(np.mean([(a + 1) * gu_bytes for a in act]))
        achieved = per_launch / (avg_us * 1e-6) / 1e9
        tb = measured_traffic() if args.workload == "bat80" and args.path != 1 else None
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if tb is None else round(tb / (avg_us * 1e-6) / 1e9, 1),
                "kernel": f"k_gateup_tiles ({wname} gate/up + SwiGLU)" if grouped else
                          f"k_gateup_gemv ({wname} gate/up partial sums)",
                "avg_us": round(avg_us, 2), "bytes_per_launch": int(per_launch),
                "traffic_bytes_per_launch": None if tb is None else int(tb),
                "events": "HIP events on the launch stream around each layer's gate/up kernel, eager replay"}
        # the other timed kernels against the same peak: down (d values and
        # their fp16 scale and bias per touched expert) and the router (the
        # E+1 fp16 router rows, plus the tokens once)
        d_bytes = (st.desc.inter * st.desc.hidden * wl.bits // 8
                   + 4 * st.desc.inter * st.desc.hidden // st.desc.group_size)
        d_launch = float(np.mean([(a + 1) * d_bytes for a in act]))
        r_launch = (wl.n_experts + 1) * wl.hidden * 2 + wl.tokens * wl.hidden * 2
        kernel_roof = {
            "gateup": {"bytes_per_launch": int(per_launch), "avg_us": round(avg_us, 2),
                       "GBps": round(achieved, 1), "frac": round(achieved / HBM_PEAK_GBS, 4)},
            "down": {"bytes_per_launch": int(d_launch), "avg_us": round(kernel_us["down"], 2),
                     "GBps": round(d_launch / (kernel_us["down"] * 1e-6) / 1e9, 1),
                     "frac": round(d_launch / (kernel_us["down"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
            "router": {"bytes_per_launch": int(r_launch), "avg_us": round(kernel_us["router"], 2),
                       "GBps": round(r_launch / (kernel_us["router"] * 1e-6) / 1e9, 1),
                       "frac": round(r_launch / (kernel_us["router"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        }
        print(f"[bench] kernel avg us: " + ", ".join(f"{k} {v:.2f}" for k, v in kernel_us.items())
              + f"; gate/up {achieved:.0f} GB/s", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on the host ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, args.cpu_seconds)

    out = {
        "metric": f"MoE-layer tokens/sec + achieved HBM GB/s on {wname} expert bytes (80B-shaped)",
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms": {"median": round(float(np.median(step_ms)), 4), "p10": round(float(np.percentile(step_ms, 10)), 4),
                    "p90": round(float(np.percentile(step_ms, 90)), 4),
                    "events": "HIP events around each step on its stream, a second pass of the same K steps"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if grouped else ("f32" if wl.bits == 8 else wl.act_dtype),
        "precision": f"{wname} weights as exact f16 matrix-core operands, activations f16, fp32 accumulate"
                     if grouped else
                     ("int8 weights times activations widened to fp32, fp32 accumulate" if wl.bits == 8 else
                      "int4 weights, bf16/f16 dot2 products, fp32 accumulate"),
        "data": "synthetic (seeded; random-init weights of the stated shapes)",
        f"{wname}_expert_GBps": round(expert_gbs, 1),
        f"{wname}_frac_of_hbm_peak": round(expert_gbs / HBM_PEAK_GBS, 4),
        "active_experts_per_layer": round(float(np.mean(act)), 2),
        "config": {"workload": f"{wl.name}: {L} layers, hidden {wl.hidden}, {wl.n_experts} experts top-{wl.top_k}, "
                               f"inter {wl.inter}, shared {wl.shared_inter}, {wname} group {wl.group}, "
                               f"{wl.tokens} tokens/step, Zipf {wl.zipf_s}",
                   "global_batch": wl.tokens, "layers": L, "path": ["auto", "gemv", "grouped"][args.path],
                   "graph": not args.eager, "parallelism": "single GPU"},
        "roofline": roof,
        "kernel_avg_us": {k: round(v, 2) for k, v in kernel_us.items()},
        "kernel_roofline": kernel_roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
