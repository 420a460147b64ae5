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
