"""HBM slot pool fed from pinned host blobs: the hit/miss/victim trace equals
the pool simulator's (own Python code), and every layer computed from the
pool's slots equals, bit for bit, the same layer computed from resident
weights (placement does not change any result)."""
import dataclasses

import numpy as np
import pytest

import synth
from oracle.pool_sim import PoolSim
from moe_testlib import DeviceLayer, desc_for

pytestmark = pytest.mark.gpu

POOLED = dataclasses.replace(synth.TINY, name="pooled", n_experts=16, top_k=3, tokens=1, layers=2,
                             weight_seed=41, token_seed=141, router_sigma=0.05, zipf_s=1.1)


@pytest.mark.parametrize("dma_copy", [False, True], ids=["copy_kernel", "copy_engine"])
def test_streamed_layers_equal_resident_and_trace_matches_simulator(dma_copy):
    import torch
    from int4_routed_expert_router_amd import api
    wl = POOLED
    L, E, K, H = wl.layers, wl.n_experts, wl.top_k, wl.hidden
    slots, period, steps = 5, 4, 14
    dls = [DeviceLayer(wl, l, use_gpu_fill=False) for l in range(L)]
    stride = dls[0].stride
    blob = api.blob_bytes(H, wl.inter, wl.group)
    host = torch.empty(L * E * stride, dtype=torch.uint8, pin_memory=True)
    for l in range(L):
        host[l * E * stride:(l + 1) * E * stride].copy_(dls[l].experts.cpu())
    slab = torch.zeros(L * slots * stride, dtype=torch.uint8, device="cuda")
    offsets = torch.zeros(L * E, dtype=torch.int64, device="cuda")
    copy_stream = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    pool = api.SlotPool(L, E, slots, period, stride, blob, host, slab, offsets, copy_stream, dma_copy=dma_copy)
    sim = PoolSim(L, E, slots, period, blob_bytes=blob)
    desc = desc_for(wl, path=1)
    ws = api.workspace(desc, 1)
    for step in range(steps):
        x_bits = synth.tokens(wl, step=step)
        x = torch.from_numpy(x_bits.view(np.int16).copy()).cuda()
        for l in range(L):
            dl = dls[l]
            idx = torch.empty(1, K, dtype=torch.int32, device="cuda")
            w = torch.empty(1, K, dtype=torch.float32, device="cuda")
            g = torch.empty(1, dtype=torch.float32, device="cuda")
            api.route(desc, dl.api_layer(), x, idx, w, g, ws=ws)
            ids = idx.cpu().numpy()[0]
            got = pool.acquire(l, ids, step, compute)
            assert got == sim.acquire(l, ids, step), f"step {step} layer {l}: pool trace differs from the simulator"
            streamed = api.Layer(dl.router_w, dl.router_bias, slab[l * slots * stride:], stride,
                                 offsets[l * E:], dl.shared)
            y_pool = torch.empty(1, H, dtype=torch.float32, device="cuda")
            y_res = torch.empty(1, H, dtype=torch.float32, device="cuda")
            api.expert_ffn(desc, streamed, x, idx, w, g, y_pool, ws=ws)
            pool.release(l, compute)
            api.expert_ffn(desc, dl.api_layer(), x, idx, w, g, y_res, ws=ws)
            torch.cuda.synchronize()
            assert np.array_equal(y_pool.cpu().numpy(), y_res.cpu().numpy()), f"step {step} layer {l}"
            sim.release(l)
    assert pool.stats() == sim.stats()
    assert sim.stats()["misses"] > slots * L and sim.stats()["evictions"] > 0
    pool.close()


@pytest.mark.parametrize("dma_copy", [False, True], ids=["copy_kernel", "copy_engine"])
def test_prefetched_layers_equal_resident_and_trace_matches_simulator(dma_copy):
    """Pre-gated prefetch: before each layer's acquire the pool prefetches a
    prediction of that layer's experts (the true set with one entry swapped,
    issued right before the acquire so that its copies are still in flight
    when the FFN is enqueued), and the next layer's experts as its own router
    predicts them from this layer's input.  Results must not change."""
    import torch
    from int4_routed_expert_router_amd import api
    wl = POOLED
    L, E, K, H = wl.layers, wl.n_experts, wl.top_k, wl.hidden
    slots, period, steps = 5, 4, 12
    dls = [DeviceLayer(wl, l, use_gpu_fill=False) for l in range(L)]
    stride = dls[0].stride
    blob = api.blob_bytes(H, wl.inter, wl.group)
    host = torch.empty(L * E * stride, dtype=torch.uint8, pin_memory=True)
    for l in range(L):
        host[l * E * stride:(l + 1) * E * stride].copy_(dls[l].experts.cpu())
    slab = torch.zeros(L * slots * stride, dtype=torch.uint8, device="cuda")
    offsets = torch.zeros(L * E, dtype=torch.int64, device="cuda")
    copy_stream = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    pool = api.SlotPool(L, E, slots, period, stride, blob, host, slab, offsets, copy_stream, dma_copy=dma_copy)
    sim = PoolSim(L, E, slots, period, blob_bytes=blob)
    desc = desc_for(wl, path=1)
    ws = api.workspace(desc, 1)
    rng = np.random.default_rng(7)
    for step in range(steps):
        x = torch.from_numpy(synth.tokens(wl, step=step).view(np.int16).copy()).cuda()
        for l in range(L):
            dl = dls[l]
            idx = torch.empty(1, K, dtype=torch.int32, device="cuda")
            w = torch.empty(1, K, dtype=torch.float32, device="cuda")
            g = torch.empty(1, dtype=torch.float32, device="cuda")
            api.route(desc, dl.api_layer(), x, idx, w, g, ws=ws)
            ids = idx.cpu().numpy()[0]
            pred = [int(e) for e in ids]
            c = int(rng.integers(0, E))
            if c not in pred:
                pred[int(rng.integers(0, K))] = c
            assert pool.prefetch(l, pred, step, compute) == sim.prefetch(l, pred, step), (step, l)
            got = pool.acquire(l, ids, step, compute)
            assert got == sim.acquire(l, ids, step), f"step {step} layer {l}: pool trace differs from the simulator"
            streamed = api.Layer(dl.router_w, dl.router_bias, slab[l * slots * stride:], stride,
                                 offsets[l * E:], dl.shared)
            y_pool = torch.empty(1, H, dtype=torch.float32, device="cuda")
            y_res = torch.empty(1, H, dtype=torch.float32, device="cuda")
            api.expert_ffn(desc, streamed, x, idx, w, g, y_pool, ws=ws)
            pool.release(l, compute)
            sim.release(l)
            # pre-gating of the next layer: its router applied to this layer's input
            if l + 1 < L:
                nxt = dls[l + 1]
                pidx = torch.empty(1, K, dtype=torch.int32, device="cuda")
                api.route(desc, nxt.api_layer(), x, pidx, w.clone(), g.clone(), ws=ws)
                p_ids = pidx.cpu().numpy()[0]
                assert pool.prefetch(l + 1, p_ids, step, compute) == sim.prefetch(l + 1, p_ids, step)
            api.expert_ffn(desc, dl.api_layer(), x, idx, w, g, y_res, ws=ws)
            torch.cuda.synchronize()
            assert np.array_equal(y_pool.cpu().numpy(), y_res.cpu().numpy()), f"step {step} layer {l}"
    st = pool.stats()
    assert st == sim.stats()
    assert st["prefetches"] > 0 and st["hits"] > 0
    pool.close()


POOLED4 = dataclasses.replace(POOLED, name="pooled4", layers=4, weight_seed=42, token_seed=142)


@pytest.mark.parametrize("pregate", [0, 2, 3], ids=["demand_only", "pregate_top2", "pregate_all"])
def test_native_pool_decode_equals_resident_stack(pregate):
    """moe_pool_decode_step (the native per-token loop over the layers) gives,
    bit for bit, the resident stack's residual, next input and selections, and
    its pool trace (selections and pre-gated predictions logged by the call)
    replays on the simulator to the same statistics."""
    import torch
    from int4_routed_expert_router_amd import api
    wl = POOLED4
    L, E, K, H = wl.layers, wl.n_experts, wl.top_k, wl.hidden
    slots, period, steps = 5, 4, 10
    dls = [DeviceLayer(wl, l, use_gpu_fill=False) for l in range(L)]
    stride = dls[0].stride
    blob = api.blob_bytes(H, wl.inter, wl.group)
    host = torch.empty(L * E * stride, dtype=torch.uint8, pin_memory=True)
    for l in range(L):
        host[l * E * stride:(l + 1) * E * stride].copy_(dls[l].experts.cpu())
    slab = torch.zeros(L * slots * stride, dtype=torch.uint8, device="cuda")
    offsets = torch.zeros(L * E, dtype=torch.int64, device="cuda")
    copy_stream = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    pool = api.SlotPool(L, E, slots, period, stride, blob, host, slab, offsets, copy_stream)
    sim = PoolSim(L, E, slots, period, blob_bytes=blob)
    desc = desc_for(wl, path=1)
    ws = api.workspace(desc, 1)
    ws_ref = api.workspace(desc, 1)
    layers = [dl.api_layer() for dl in dls]
    idx_host = torch.empty(2, K, dtype=torch.int32, pin_memory=True)
    x_buf = torch.empty(2, H, dtype=torch.int16, device="cuda")
    for step in range(steps):
        x_bits = synth.tokens(wl, step=step)
        x0 = torch.from_numpy(x_bits.view(np.int16).copy()).cuda()
        r0 = x0.view(torch.float16).float() if wl.act_dtype == "f16" else x0.view(torch.bfloat16).float()
        r = r0.clone()
        log = np.zeros((L, 2, K), np.int32)
        api.pool_decode_step(desc, layers, pool, step, x0, r, x_buf, idx_host, ws, pregate=pregate, idx_log=log,
                             stream=compute)
        r_ref = r0.clone()
        xb_ref = torch.empty_like(x0)
        idx_all = torch.empty(L, 1, K, dtype=torch.int32, device="cuda")
        api.stack_forward(desc, layers, x0, r_ref, xb_ref, ws_ref, idx_all=idx_all)
        torch.cuda.synchronize()
        assert np.array_equal(r.cpu().numpy(), r_ref.cpu().numpy()), f"step {step}: residual differs"
        assert np.array_equal(x_buf[(L - 1) % 2].cpu().numpy(), xb_ref[0].cpu().numpy()), f"step {step}"
        assert np.array_equal(log[:, 0], idx_all.cpu().numpy()[:, 0]), f"step {step}: selections differ"
        for l in range(L):
            sim.acquire(l, log[l, 0], step)
            if pregate and l + 1 < L:
                assert (log[l, 1, pregate:] == -1).all() and (log[l, 1, :pregate] >= 0).all()
                sim.prefetch(l + 1, log[l, 1, :pregate], step)
            else:
                assert (log[l, 1] == -1).all()
            sim.release(l)
    assert pool.stats() == sim.stats()
    assert (pool.stats()["prefetches"] > 0) == (pregate > 0)
    pool.close()


def test_native_pool_decode_rejects_a_pool_of_other_geometry():
    import torch
    from int4_routed_expert_router_amd import api, MoeError
    wl = POOLED4
    dl = DeviceLayer(wl, 0, use_gpu_fill=False)
    stride = dl.stride
    host = torch.empty(8 * stride, dtype=torch.uint8, pin_memory=True)
    slab = torch.zeros(4 * stride, dtype=torch.uint8, device="cuda")
    offsets = torch.zeros(8, dtype=torch.int64, device="cuda")
    pool = api.SlotPool(1, 8, 4, 0, stride, stride, host, slab, offsets, torch.cuda.Stream())   # 8 experts, not 16
    desc = desc_for(wl, path=1)
    x = torch.zeros(1, wl.hidden, dtype=torch.int16, device="cuda")
    r = torch.zeros(wl.hidden, dtype=torch.float32, device="cuda")
    xb = torch.empty(2, wl.hidden, dtype=torch.int16, device="cuda")
    idx_host = torch.empty(2, wl.top_k, dtype=torch.int32, pin_memory=True)
    with pytest.raises(MoeError, match="MOE_ESHAPE"):
        api.pool_decode_step(desc, [dl.api_layer()], pool, 0, x, r, xb, idx_host, api.workspace(desc, 1))
    pool.close()
