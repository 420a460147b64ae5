"""Parity at the widths the benchmark runs: the 80B-shaped stacks (hidden
2048, 512 experts, top-10, inter 512) chained through the residual epilogue
and replayed from a captured HIP graph, the pooled decode at that shape,
batch invariance of the batched layer, the shape-specialised grouped kernels
without a shared expert and with down ranges over three units, and the fp16
range status of the grouped family.

The pages' validation paragraph (Show HN page) names the checks adapted
here: decoding token by token agrees with running the batch at once (batch
invariance), and an expert gives the same result wherever it was loaded
from (placement invariance of the pooled decode)."""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import moe_oracle as mo
from oracle.pool_sim import PoolSim
from moe_testlib import DeviceLayer, assert_close, check_routing, desc_for
from test_gpu_stack import oracle_sets

pytestmark = pytest.mark.gpu


class FullStack:
    """L layers of a 2048-wide workload with distinct weights (generated on the
    GPU), run eagerly and from a captured graph, with per-layer captures."""

    def __init__(self, wl, n_layers, n_tokens, path=0):
        import torch
        from int4_routed_expert_router_amd import api
        self.wl, self.L, self.T = wl, n_layers, n_tokens
        self.desc = desc_for(wl, path=path)
        self.dl = [DeviceLayer(wl, l) for l in range(n_layers)]
        self.layers = [d.api_layer() for d in self.dl]
        self.x0_bits = synth.tokens(wl, n_tokens=n_tokens)
        self.x0 = torch.from_numpy(self.x0_bits.view(np.int16).copy()).cuda()
        self.r0 = torch.from_numpy(mo.act_bits_to_f64(self.x0_bits, wl.act_dtype).astype(np.float32)).cuda()
        L, T, H, K = n_layers, n_tokens, wl.hidden, wl.top_k
        self.r = self.r0.clone()
        self.x_buf = torch.empty_like(self.x0)
        self.ws = api.workspace(self.desc, T)
        self.x_all = torch.empty(L, T, H, dtype=torch.int16, device="cuda")
        self.y_all = torch.empty(L, T, H, dtype=torch.float32, device="cuda")
        self.idx_all = torch.empty(L, T, K, dtype=torch.int32, device="cuda")
        self.w_all = torch.empty(L, T, K, dtype=torch.float32, device="cuda")
        self.g_all = torch.empty(L, T, dtype=torch.float32, device="cuda")

    def captures(self):
        return dict(x_all=self.x_all, y_all=self.y_all, idx_all=self.idx_all, w_all=self.w_all,
                    gamma_all=self.g_all)

    def snapshot(self):
        return {k: v.cpu().numpy().copy() for k, v in dict(r=self.r, **self.captures()).items()}

    def run_eager(self):
        import torch
        from int4_routed_expert_router_amd import api
        self.r.copy_(self.r0)
        api.stack_forward(self.desc, self.layers, self.x0, self.r, self.x_buf, self.ws, **self.captures())
        torch.cuda.synchronize()
        return self.snapshot()

    def run_graph(self, replays):
        """Replays of one captured graph, with the program's own eager work
        between them; returns one snapshot per replay."""
        import torch
        from int4_routed_expert_router_amd import api
        stream = torch.cuda.Stream()
        g = api.StackGraph(self.desc, self.layers, self.x0, self.r, self.x_buf, self.ws, stream, **self.captures())
        snaps = []
        for _ in range(replays):
            self.y_all.fill_(float("nan"))
            self.idx_all.fill_(-1)
            self.r.copy_(self.r0)
            torch.cuda.synchronize()
            g.launch(stream)
            torch.cuda.synchronize()
            snaps.append(self.snapshot())
        g.close()
        return snaps


def teacher_forced(st, got):
    """Each layer against the oracle on the GPU's own input of that layer;
    the epilogue's next input within one bf16 ulp; the final residual."""
    wl = st.wl
    r = mo.act_bits_to_f64(st.x0_bits, wl.act_dtype)
    flagged = 0
    for l in range(st.L):
        x_bits = got["x_all"][l].view(np.uint16)
        if l == 0:
            assert np.array_equal(x_bits, st.x0_bits)
        x64 = mo.act_bits_to_f64(x_bits, wl.act_dtype)
        dl = st.dl[l]
        sets, fl = oracle_sets(x64, dl.router_f64(), dl.bias_f64(), got["idx_all"][l], wl.top_k)
        flagged += fl
        ref = mo.layer_forward(x64, dl.router_f64(), dl.bias_f64(), dl.oracle_expert, dl.oracle_shared(), wl.top_k,
                               forced_idx=sets)
        assert_close(got["w_all"][l], ref["w"], f"layer {l} routing weights")
        assert_close(got["gamma_all"][l], ref["gamma"], f"layer {l} shared gate")
        worst, tol = assert_close(got["y_all"][l], ref["y"], f"layer {l} output")
        print(f"{wl.name} layer {l}: max err {worst:.3e} (tol {tol:.3e})")
        r, x_next = mo.stack_epilogue(r, got["y_all"][l].astype(np.float64))
        if l + 1 < st.L:
            nxt = got["x_all"][l + 1].view(np.uint16).astype(np.int64)
            diff = np.abs(nxt - x_next.astype(np.int64))
            assert diff.max() <= 1, f"layer {l} epilogue differs by {diff.max()} bf16 ulps"
        dl._cache.clear()
    assert_close(got["r"], r, "final residual")
    return flagged


@pytest.mark.parametrize("wl_name,n_tokens", [("bat80", 64), ("dec80", 1), ("dec35", 1), ("dec80i8", 1)])
def test_chained_stack_graph_replay_parity(wl_name, n_tokens):
    """Three chained layers at the benchmarks' shapes (batched: grouped family
    with the fused combine + epilogue at hidden 2048; batch 1: GEMV family
    with top-K inside gate/up, at the 80B and 35B shapes and with int8
    experts), replayed from one captured graph twice:
    every replay equals the eager run bit for bit, and each layer matches the
    oracle (teacher forced)."""
    wl = synth.WORKLOADS[wl_name]
    st = FullStack(wl, 3, n_tokens)
    want = st.run_eager()
    for rep, got in enumerate(st.run_graph(2)):
        for k in want:
            assert np.array_equal(got[k], want[k]), f"replay {rep}: {k} differs from the eager run"
    flagged = teacher_forced(st, want)
    print(f"{wl_name}: near ties {flagged}")


def test_pooled_decode_at_the_80b_shape_equals_resident():
    """The native pooled decode (128 HBM slots per layer = 25% of 512 experts,
    blobs in pinned host memory) gives, bit for bit, the resident stack's
    residual and selections for every token, with misses and evictions, and
    its trace replays on the pool simulator to the same statistics."""
    import torch
    from int4_routed_expert_router_amd import api
    wl = dataclasses.replace(synth.POOL80, layers=3)
    L, E, K, H, S = wl.layers, wl.n_experts, wl.top_k, wl.hidden, wl.slots_per_layer
    steps, period = 40, 8
    dls = [DeviceLayer(wl, l) for l in range(L)]
    stride = dls[0].stride
    blob = api.blob_bytes(H, wl.inter, wl.group)
    host = torch.empty(L * E * stride, dtype=torch.uint8, pin_memory=True)
    for l in range(L):
        host[l * E * stride:(l + 1) * E * stride].copy_(dls[l].experts.cpu())
    slab = torch.zeros(L * S * stride, dtype=torch.uint8, device="cuda")
    offsets = torch.zeros(L * E, dtype=torch.int64, device="cuda")
    compute = torch.cuda.current_stream()
    pool = api.SlotPool(L, E, S, period, stride, blob, host, slab, offsets, torch.cuda.Stream())
    sim = PoolSim(L, E, S, period, blob_bytes=blob)
    desc = desc_for(wl, path=0)
    ws, ws_ref = api.workspace(desc, 1), api.workspace(desc, 1)
    resident = [dl.api_layer() for dl in dls]
    pooled = [api.Layer(dl.router_w, dl.router_bias, slab, stride, offsets, dl.shared) for dl in dls]
    idx_host = torch.empty(2, K, dtype=torch.int32, pin_memory=True)
    x_buf = torch.empty(2, H, dtype=torch.int16, device="cuda")
    for step in range(steps):
        x0 = torch.from_numpy(synth.tokens(wl, step=step).view(np.int16).copy()).cuda()
        r0 = x0.view(torch.bfloat16).float()
        r = r0.clone()
        log = np.zeros((L, 2, K), np.int32)
        api.pool_decode_step(desc, pooled, pool, step, x0, r, x_buf, idx_host, ws, idx_log=log, stream=compute)
        r_ref = r0.clone()
        xb_ref = torch.empty_like(x0)
        idx_all = torch.empty(L, 1, K, dtype=torch.int32, device="cuda")
        api.stack_forward(desc, resident, x0, r_ref, xb_ref, ws_ref, idx_all=idx_all)
        torch.cuda.synchronize()
        assert np.array_equal(r.cpu().numpy(), r_ref.cpu().numpy()), f"step {step}: residual differs"
        assert np.array_equal(log[:, 0], idx_all.cpu().numpy()[:, 0]), f"step {step}: selections differ"
        for l in range(L):
            sim.acquire(l, log[l, 0], step)
            sim.release(l)
    st = pool.stats()
    assert st == sim.stats()
    assert st["misses"] > S and st["evictions"] > 0, st
    print(f"pooled 80B shape: {st}")
    pool.close()


def test_batch_invariance_of_the_batched_layer():
    """64 tokens in one call (grouped matrix-core family, matrix-core router)
    against the same 64 tokens one call each (GEMV family, per-row router):
    identical expert indices, outputs within the oracle tolerance of each
    other."""
    import torch
    from int4_routed_expert_router_amd import api
    wl = synth.BAT80
    dl = DeviceLayer(wl, 9)
    desc = desc_for(wl)
    T, K, H = wl.tokens, wl.top_k, wl.hidden
    x = torch.from_numpy(synth.tokens(wl).view(np.int16).copy()).cuda()
    y = torch.empty(T, H, dtype=torch.float32, device="cuda")
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    api.layer_forward(desc, dl.api_layer(), x, y, idx, w)
    y1 = torch.empty(T, H, dtype=torch.float32, device="cuda")
    idx1 = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w1 = torch.empty(T, K, dtype=torch.float32, device="cuda")
    ws1 = api.workspace(desc, 1)
    for t in range(T):
        api.layer_forward(desc, dl.api_layer(), x[t:t + 1], y1[t:t + 1], idx1[t:t + 1], w1[t:t + 1], ws=ws1)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), idx1.cpu().numpy()), "batched and single-token selections differ"
    assert_close(w.cpu().numpy(), w1.cpu().numpy(), "routing weights, batched vs one token per call")
    worst, tol = assert_close(y.cpu().numpy(), y1.cpu().numpy(), "output, batched vs one token per call")
    print(f"batch invariance: max |batched - single| {worst:.3e} (tol {tol:.3e})")


def sampled_layer_check(wl, layer, x_bits, path, sample, shared=True):
    """The layer on all tokens on the GPU; the oracle on the sampled tokens
    (each token's output depends on its own routing only)."""
    import torch
    from int4_routed_expert_router_amd import api
    dl = DeviceLayer(wl, layer)
    desc = desc_for(wl, path=path, shared_inter=None if shared else 0)
    T, K, H, E = x_bits.shape[0], wl.top_k, wl.hidden, wl.n_experts
    x = torch.from_numpy(x_bits.view(np.int16).copy()).cuda()
    y = torch.empty(T, H, dtype=torch.float32, device="cuda")
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    logits = torch.empty(T, E + 1, dtype=torch.float32, device="cuda")
    ws = api.workspace(desc, T)
    api.route(desc, dl.api_layer(), x, idx, w, None, logits, ws=ws)
    api.layer_forward(desc, dl.api_layer(), x, y, ws=ws)
    torch.cuda.synchronize()
    assert api.workspace_status(desc, T, ws) == 0
    g_idx, g_w, g_lg, g_y = (t.cpu().numpy() for t in (idx, w, logits, y))
    x64 = mo.act_bits_to_f64(x_bits[sample], wl.act_dtype)
    sets, flagged = check_routing(g_idx[sample], g_w[sample], g_lg[sample], x64, dl.router_f64(), dl.bias_f64(), K)
    ref = mo.layer_forward(x64, dl.router_f64(), dl.bias_f64(), dl.oracle_expert,
                           dl.oracle_shared() if shared else None, K, forced_idx=sets)
    assert_close(g_w[sample], ref["w"], "routing weights (sample)")
    worst, tol = assert_close(g_y[sample], ref["y"], f"{wl.name} T={T} output (sample)")
    assert np.isfinite(g_y).all()
    return worst, tol, flagged


def test_grouped_full_shape_without_shared_expert():
    # the shape-specialised grouped kernels with shared_inter = 0 (no shared
    # units: the unit list starts at the routed experts)
    wl = synth.BAT80
    x_bits = synth.tokens(wl)
    worst, tol, _ = sampled_layer_check(wl, 13, x_bits, 2, np.arange(wl.tokens), shared=False)
    print(f"bat80 shape, no shared expert: max err {worst:.3e} (tol {tol:.3e})")


def test_grouped_full_shape_down_ranges_over_three_units():
    # 1024 tokens at the 2048/512 shape: about 700 units of 16 rows, 16 down
    # quads each, so a down workgroup's range of about 44 quads spans three or
    # four units and restages h into a buffer it used two units before
    wl = synth.BAT80
    T = 1024
    x_bits = synth.tokens(wl, n_tokens=T, seed=wl.token_seed + T)
    sample = np.unique(np.concatenate([np.arange(0, T, 37), [T - 1]]))
    worst, tol, flagged = sampled_layer_check(wl, 17, x_bits, 2, sample)
    print(f"bat80 shape, {T} tokens, {len(sample)} sampled: max err {worst:.3e} (tol {tol:.3e}), near ties {flagged}")


def test_fp16_range_status_of_the_grouped_family():
    """Activations or SwiGLU outputs beyond the fp16 operand range set
    MOE_FLAG_F16_RANGE in the call's status word; in-range batches leave it
    clear; the GEMV family runs the same tokens with finite results and
    reports nothing, and its in-range tokens keep the oracle tolerance (the
    tolerance is a statement about the workloads' activation scale, so the
    token at 300 times that scale is only required to be finite)."""
    import torch
    from int4_routed_expert_router_amd import api
    from int4_routed_expert_router_amd._lib import MOE_FLAG_F16_RANGE
    wl = synth.BAT80
    dl = DeviceLayer(wl, 21)
    T, H = wl.tokens, wl.hidden
    base = mo.bf16_bits_to_f64(synth.tokens(wl))

    def run(x64, path):
        desc = desc_for(wl, path=path)
        n = x64.shape[0]
        x = torch.from_numpy(mo.f64_to_bf16_bits_rne(x64).view(np.int16).copy()).cuda()
        y = torch.empty(n, H, dtype=torch.float32, device="cuda")
        ws = api.workspace(desc, n)
        ws.fill_(0xFF)                      # stale contents: the call must clear the word
        api.layer_forward(desc, dl.api_layer(), x, y, ws=ws)
        torch.cuda.synchronize()
        return api.workspace_status(desc, n, ws), y.cpu().numpy()

    st, _ = run(base, 2)
    assert st == 0
    big_x = base.copy()
    big_x[5] *= 1e5                         # activations beyond 65520
    st, _ = run(big_x, 2)
    assert st & MOE_FLAG_F16_RANGE
    big_h = base.copy()
    big_h[11] *= 300.0                      # activations in range, h = silu(a) u beyond it
    assert np.abs(big_h).max() < 65504
    st, _ = run(big_h, 2)
    assert st & MOE_FLAG_F16_RANGE
    st, y = run(big_h[8:12], 1)             # GEMV family: no fp16 operands
    assert st == 0 and np.isfinite(y).all()
    x64 = big_h[8:11]
    ref = mo.layer_forward(x64, dl.router_f64(), dl.bias_f64(), dl.oracle_expert, dl.oracle_shared(), wl.top_k)
    assert_close(y[:3], ref["y"], "GEMV family, in-range tokens of the batch")
