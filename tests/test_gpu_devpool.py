"""GPU-resident slot pool: the policy kernel's trace equals the pool simulator's
(own Python code) request by request, the streamed decode (no host round
trip per layer; on the GEMV family the gate/up kernel copies the misses
beside its products, a missed expert's rows waiting for its sections)
equals the resident stack bit for bit with no wait given up, and the
captured token graph replays token after token with the step advancing on
the device.  The pages' placement check: an expert gives the same result whether it
was already resident or had to be loaded (Show HN page, validation
paragraph)."""
import dataclasses

import numpy as np
import pytest

import synth
from oracle.pool_sim import PoolSim
from moe_testlib import DeviceLayer, desc_for

pytestmark = pytest.mark.gpu

POOLED4 = dataclasses.replace(synth.TINY, name="pooled4", n_experts=16, top_k=3, tokens=1, layers=4,
                              weight_seed=42, token_seed=142, router_sigma=0.05, zipf_s=1.1)


class DevPoolRig:
    def __init__(self, wl, slots, period, path=0):
        import torch
        from int4_routed_expert_router_amd import api
        self.wl = wl
        L, E, H = wl.layers, wl.n_experts, wl.hidden
        self.dls = [DeviceLayer(wl, l, use_gpu_fill=wl.hidden > 256) for l in range(L)]
        self.stride = self.dls[0].stride
        self.blob = api.blob_bytes(H, wl.inter, wl.group, wl.bits)
        self.host = torch.empty(L * E * self.stride, dtype=torch.uint8, pin_memory=True)
        for l in range(L):
            self.host[l * E * self.stride:(l + 1) * E * self.stride].copy_(self.dls[l].experts.cpu())
        self.slots, self.period = slots, period
        self.desc = desc_for(wl, path=path)
        self.layers = [dl.api_layer() for dl in self.dls]

    def pool(self):
        import torch
        from int4_routed_expert_router_amd import api
        wl = self.wl
        slab = torch.zeros(wl.layers * self.slots * self.stride, dtype=torch.uint8, device="cuda")
        offsets = torch.zeros(wl.layers * wl.n_experts, dtype=torch.int64, device="cuda")
        return api.DevPool(wl.layers, wl.n_experts, self.slots, self.period, self.stride, self.blob, self.host, slab,
                           offsets)

    def resident(self, x0):
        """The resident stack on one token: residual, next input, selections."""
        import torch
        from int4_routed_expert_router_amd import api
        wl = self.wl
        r = x0.view(torch.bfloat16).float() if wl.act_dtype == "bf16" else x0.view(torch.float16).float()
        r = r.reshape(-1).contiguous()
        xb = torch.empty_like(x0)
        idx_all = torch.empty(wl.layers, 1, wl.top_k, dtype=torch.int32, device="cuda")
        api.stack_forward(self.desc, self.layers, x0, r, xb, api.workspace(self.desc, 1), idx_all=idx_all)
        torch.cuda.synchronize()
        return r.cpu().numpy(), xb[0].cpu().numpy(), idx_all.cpu().numpy()[:, 0]


def check_trace(sim, step, sel, trace):
    for l in range(sel.shape[0]):
        want = sim.acquire(l, sel[l], step)
        sim.release(l)
        got = [(int(e), bool(trace[l, k, 2]), int(trace[l, k, 0]), int(trace[l, k, 1])) for k, e in enumerate(sel[l])]
        assert got == want, f"step {step} layer {l}: device pool {got} != simulator {want}"


@pytest.mark.parametrize("slots,period,path,bits", [(5, 4, 0, 4), (3, 0, 0, 4), (16, 2, 0, 4), (5, 4, 2, 4),
                                                     (5, 4, 0, 8)],
                         ids=["5_slots", "3_slots_no_aging", "all_resident", "5_slots_grouped_copy_kernel",
                              "5_slots_int8"])
def test_device_pool_trace_and_placement(slots, period, path, bits):
    """path 0: the GEMV family, misses copied inside the gate/up kernel (its
    gate/up and down byte ranges of the blob, int4 or int8); path 2 (the
    grouped family forced): misses copied by the copy kernel after the
    acquire."""
    import torch
    from int4_routed_expert_router_amd import api
    from int4_routed_expert_router_amd._lib import MOE_FLAG_STREAM_WAIT
    wl = POOLED4 if bits == 4 else dataclasses.replace(POOLED4, name="pooled4_int8", bits=8, scale_lo=1e-4,
                                                       scale_hi=1e-3)
    rig = DevPoolRig(wl, slots, period, path)
    pool = rig.pool()
    sim = PoolSim(wl.layers, wl.n_experts, slots, period, blob_bytes=rig.blob)
    L, K, H = wl.layers, wl.top_k, wl.hidden
    ws = api.workspace(rig.desc, 1)
    x_buf = torch.empty(2, H, dtype=torch.int16, device="cuda")
    trace = torch.full((L, K, 3), -9, dtype=torch.int32, device="cuda")
    steps = 14
    for step in range(steps):
        x0 = torch.from_numpy(synth.tokens(wl, step=step).view(np.int16).copy()).cuda()
        r = (x0.view(torch.float16).float() if wl.act_dtype == "f16" else x0.view(torch.bfloat16).float()).reshape(-1)
        api.pool_decode_step_dev(rig.desc, rig.layers, pool, x0, r, x_buf, ws, trace=trace)
        torch.cuda.synchronize()
        assert api.workspace_status(rig.desc, 1, ws) & MOE_FLAG_STREAM_WAIT == 0, f"step {step}: a wait gave up"
        r_ref, x_ref, sel = rig.resident(x0)
        assert np.array_equal(r.cpu().numpy(), r_ref), f"step {step}: residual differs from the resident stack"
        assert np.array_equal(x_buf[(L - 1) % 2].cpu().numpy(), x_ref), f"step {step}: next input differs"
        check_trace(sim, step, sel, trace.cpu().numpy())
    st = pool.stats()
    want = sim.stats()
    assert (st["hits"], st["misses"], st["evictions"], st["bytes_h2d"]) == \
        (want["hits"], want["misses"], want["evictions"], want["bytes_h2d"])
    assert st["step"] == steps and st["error"] == 0
    if slots < wl.n_experts:
        assert st["evictions"] > 0
    pool.close()


@pytest.mark.parametrize("n_experts,top_k,slots,period", [(300, 16, 200, 4), (350, 32, 300, 0), (700, 64, 600, 3)],
                         ids=["4_slots_per_lane", "8_slots_per_lane", "16_slots_per_lane_E700_K64"])
def test_device_pool_larger_pools(n_experts, top_k, slots, period):
    """The policy kernel is instantiated per slots per lane (1, 2, 4, 8, 16)
    and selects the token's experts itself (8 or 16 logits per lane): pools
    of 200 to 600 slots per layer, up to 64 experts per token, trace equal to
    the pool simulator's and the streamed stack equal to the resident one."""
    import torch
    from int4_routed_expert_router_amd import api
    wl = dataclasses.replace(synth.TINY, name="pooled_big", hidden=64, inter=64, shared_inter=64, group=32,
                             n_experts=n_experts, top_k=top_k, tokens=1, layers=2, weight_seed=43, token_seed=143,
                             router_sigma=0.5, zipf_s=0.0)   # diverse selections, so the pools fill and evict
    rig = DevPoolRig(wl, slots, period)
    pool = rig.pool()
    sim = PoolSim(wl.layers, wl.n_experts, slots, period, blob_bytes=rig.blob)
    L, K, H = wl.layers, wl.top_k, wl.hidden
    ws = api.workspace(rig.desc, 1)
    x_buf = torch.empty(2, H, dtype=torch.int16, device="cuda")
    trace = torch.full((L, K, 3), -9, dtype=torch.int32, device="cuda")
    steps = 24
    for step in range(steps):
        x0 = torch.from_numpy(synth.tokens(wl, step=step).view(np.int16).copy()).cuda()
        r = x0.view(torch.float16).float().reshape(-1)
        api.pool_decode_step_dev(rig.desc, rig.layers, pool, x0, r, x_buf, ws, trace=trace)
        torch.cuda.synchronize()
        r_ref, x_ref, sel = rig.resident(x0)
        assert np.array_equal(r.cpu().numpy(), r_ref), f"step {step}: residual differs from the resident stack"
        check_trace(sim, step, sel, trace.cpu().numpy())
    st = pool.stats()
    want = sim.stats()
    assert (st["hits"], st["misses"], st["evictions"]) == (want["hits"], want["misses"], want["evictions"])
    assert st["evictions"] > 0 and st["error"] == 0, st
    pool.close()


def test_device_pool_graph_replays_token_after_token():
    """One captured token graph launched once per token (the input copied into
    the captured x0 buffer between launches): the same residuals, next inputs
    and traces as the eager device-pool calls on a second pool."""
    import torch
    from int4_routed_expert_router_amd import api
    wl = POOLED4
    rig = DevPoolRig(wl, 5, 4)
    L, K, H = wl.layers, wl.top_k, wl.hidden
    pg, pe = rig.pool(), rig.pool()
    x0 = torch.empty(1, H, dtype=torch.int16, device="cuda")
    r_g = torch.empty(H, dtype=torch.float32, device="cuda")
    xb_g = torch.empty(2, H, dtype=torch.int16, device="cuda")
    tr_g = torch.empty(L, K, 3, dtype=torch.int32, device="cuda")
    ws_g = api.workspace(rig.desc, 1)
    stream = torch.cuda.Stream()
    graph = api.PoolGraph(rig.desc, rig.layers, pg, x0, r_g, xb_g, ws_g, stream, trace=tr_g)
    xb_e = torch.empty(2, H, dtype=torch.int16, device="cuda")
    tr_e = torch.empty(L, K, 3, dtype=torch.int32, device="cuda")
    ws_e = api.workspace(rig.desc, 1)
    for step in range(10):
        tok = torch.from_numpy(synth.tokens(wl, step=step).view(np.int16).copy()).cuda()
        r0 = (tok.view(torch.float16).float() if wl.act_dtype == "f16" else tok.view(torch.bfloat16).float()).reshape(-1)
        x0.copy_(tok)
        r_g.copy_(r0)
        torch.cuda.synchronize()
        graph.launch(stream)
        r_e = r0.clone()
        api.pool_decode_step_dev(rig.desc, rig.layers, pe, tok, r_e, xb_e, ws_e, trace=tr_e)
        torch.cuda.synchronize()
        assert np.array_equal(r_g.cpu().numpy(), r_e.cpu().numpy()), f"token {step}: residual"
        assert np.array_equal(xb_g.cpu().numpy()[(L - 1) % 2], xb_e.cpu().numpy()[(L - 1) % 2]), f"token {step}"
        assert np.array_equal(tr_g.cpu().numpy(), tr_e.cpu().numpy()), f"token {step}: trace"
    assert pg.stats() == pe.stats()
    assert pg.stats()["step"] == 10
    graph.close()
    pg.close()
    pe.close()


def test_device_pool_at_the_80b_shape():
    """128 slots per layer (25% of 512 experts) at the 80B shape, 3 layers, 40
    tokens: bitwise equal to the resident stack, trace equal to the
    simulator's, with misses and evictions."""
    import torch
    from int4_routed_expert_router_amd import api
    from int4_routed_expert_router_amd._lib import MOE_FLAG_STREAM_WAIT
    wl = dataclasses.replace(synth.POOL80, layers=3)
    rig = DevPoolRig(wl, wl.slots_per_layer, 8)
    pool = rig.pool()
    sim = PoolSim(wl.layers, wl.n_experts, wl.slots_per_layer, 8, blob_bytes=rig.blob)
    L, K, H = wl.layers, wl.top_k, wl.hidden
    ws = api.workspace(rig.desc, 1)
    x_buf = torch.empty(2, H, dtype=torch.int16, device="cuda")
    trace = torch.empty(L, K, 3, dtype=torch.int32, device="cuda")
    for step in range(40):
        x0 = torch.from_numpy(synth.tokens(wl, step=step).view(np.int16).copy()).cuda()
        r = x0.view(torch.bfloat16).float().reshape(-1)
        api.pool_decode_step_dev(rig.desc, rig.layers, pool, x0, r, x_buf, ws, trace=trace)
        torch.cuda.synchronize()
        assert api.workspace_status(rig.desc, 1, ws) & MOE_FLAG_STREAM_WAIT == 0, f"step {step}: a wait gave up"
        r_ref, x_ref, sel = rig.resident(x0)
        assert np.array_equal(r.cpu().numpy(), r_ref), f"step {step}: residual differs"
        check_trace(sim, step, sel, trace.cpu().numpy())
    st = pool.stats()
    assert st["misses"] > wl.slots_per_layer and st["evictions"] > 0, st
    assert st["misses"] == sim.stats()["misses"] and st["evictions"] == sim.stats()["evictions"]
    print(f"device pool, 80B shape: {st}")
    pool.close()


def test_device_pool_rejects_bad_ids_without_changes():
    import torch
    from int4_routed_expert_router_amd import api
    wl = POOLED4
    rig = DevPoolRig(wl, 5, 4)
    slab = torch.zeros(wl.layers * 5 * rig.stride, dtype=torch.uint8, device="cuda")
    offsets = torch.zeros(wl.layers * wl.n_experts, dtype=torch.int64, device="cuda")
    pool = api.DevPool(wl.layers, wl.n_experts, 5, 4, rig.stride, rig.blob, rig.host, slab, offsets)
    # a good acquire on layer 0 leaves a miss list; a rejected one on layer 1
    # must copy nothing (its copy kernel sees an empty list, not layer 0's)
    pool.acquire(0, torch.tensor([3, 4, 2], dtype=torch.int32, device="cuda"))
    pool.acquire(1, torch.tensor([5, 5, 6], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert pool.stats()["error"] == 1
    assert int(slab[5 * rig.stride:10 * rig.stride].count_nonzero()) == 0, "a rejected acquire copied blobs"
    assert int(slab[:5 * rig.stride].count_nonzero()) > 0
    pool.reset()
    pool.acquire(0, torch.tensor([1, 1, 2], dtype=torch.int32, device="cuda"))   # repeated id
    st = pool.stats()
    assert st["error"] == 1 and st["hits"] == 0 and st["misses"] == 0
    pool.reset()
    pool.acquire(0, torch.tensor([3, 99, 2], dtype=torch.int32, device="cuda"))  # out of range
    st = pool.stats()
    assert st["error"] == 1 and st["misses"] == 0
    pool.reset()
    pool.acquire(0, torch.tensor([3, 4, 2], dtype=torch.int32, device="cuda"), bump_step=True)
    assert pool.stats() == dict(hits=0, misses=3, evictions=0, bytes_h2d=3 * rig.blob, prefetches=0, step=1, error=0)
    pool.close()
