"""The stack step: layers chained through the residual epilogue, eager and as
one captured HIP graph.  Parity is per layer with teacher forcing: the oracle
of layer l reads the GPU's own input x_l, so index flips never compound."""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import moe_oracle as mo
from moe_testlib import DeviceLayer, assert_close, desc_for

pytestmark = pytest.mark.gpu

STACK = dataclasses.replace(synth.TINY, name="stack", hidden=320, n_experts=24, top_k=3, inter=192,
                            shared_inter=128, group=64, tokens=40, layers=3, act_dtype="bf16", weight_seed=31,
                            token_seed=131, scale_lo=0.001, scale_hi=0.01, router_sigma=0.056, zipf_s=1.1)


class Stack:
    def __init__(self, wl, n_tokens, path):
        import torch
        from int4_routed_expert_router_amd import api
        self.wl, self.T = wl, n_tokens
        self.desc = desc_for(wl, path=path)
        self.dl = [DeviceLayer(wl, l, use_gpu_fill=False) for l in range(wl.layers)]
        self.layers = [d.api_layer() for d in self.dl]
        self.x0_bits = synth.tokens(wl, n_tokens=n_tokens)
        self.x0 = torch.from_numpy(self.x0_bits.view(np.int16).copy()).cuda()
        self.r0 = torch.from_numpy(mo.act_bits_to_f64(self.x0_bits, wl.act_dtype).astype(np.float32)).cuda()
        L, T, H, K = wl.layers, n_tokens, wl.hidden, wl.top_k
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

    def run_eager(self):
        import torch
        from int4_routed_expert_router_amd import api
        self.r.copy_(self.r0)
        api.stack_forward(self.desc, self.layers, self.x0, self.r, self.x_buf, self.ws, **self.captures())
        torch.cuda.synchronize()

    def snapshot(self):
        return {k: v.cpu().numpy().copy() for k, v in dict(r=self.r, **self.captures()).items()}


def oracle_sets(x64, wr64, b64, gpu_idx, k):
    """The GPU's index sets where they agree with the fp64 oracle, else only
    at near ties (gap within the fp32 logit error bound); returns the sets the
    oracle evaluates and the number of near-tie tokens."""
    z64, _ = mo.router_logits(x64, wr64, b64)
    sets, flagged = [], 0
    for t in range(x64.shape[0]):
        ref = mo.topk_order(z64[t], k)
        got = gpu_idx[t].astype(np.int64)
        if ref.tolist() != got.tolist():
            for a, b in zip(ref.tolist(), got.tolist()):
                if a != b:
                    gap = abs(z64[t, a] - z64[t, b])
                    eb = mo.logit_error_bound(x64[t], wr64, b64, a) + mo.logit_error_bound(x64[t], wr64, b64, b)
                    assert gap <= eb, f"token {t}: {a} vs {b}, gap {gap:.3e} > bound {eb:.3e}"
            flagged += 1
        sets.append(got)
    return np.stack(sets), flagged


# int8 experts: 12 tokens x 3 rows are past the GEMV row limit, so AUTO runs
# them on the grouped matrix-core family
STACK8 = dataclasses.replace(STACK, name="stack_i8", bits=8, scale_lo=1e-4, scale_hi=1e-3, weight_seed=32)


@pytest.mark.parametrize("path,n_tokens,wl", [(1, 3, STACK), (2, 40, STACK), (0, 12, STACK8)],
                         ids=["gemv", "grouped", "auto_int8"])
def test_stack_teacher_forced_parity(path, n_tokens, wl):
    st = Stack(wl, n_tokens, path)
    st.run_eager()
    got = st.snapshot()
    r = mo.act_bits_to_f64(st.x0_bits, wl.act_dtype)
    for l in range(wl.layers):
        x_bits = got["x_all"][l].view(np.uint16)
        if l == 0:
            assert np.array_equal(x_bits, st.x0_bits)
        x64 = mo.act_bits_to_f64(x_bits, wl.act_dtype)
        dl = st.dl[l]
        sets, _ = oracle_sets(x64, dl.router_f64(), dl.bias_f64(), got["idx_all"][l], wl.top_k)
        ref = mo.layer_forward(x64, dl.router_f64(), dl.bias_f64(), dl.oracle_expert, dl.oracle_shared(), wl.top_k,
                               forced_idx=sets)
        assert_close(got["w_all"][l], ref["w"], f"layer {l} routing weights")
        assert_close(got["gamma_all"][l], ref["gamma"], f"layer {l} shared gate")
        assert_close(got["y_all"][l], ref["y"], f"layer {l} output")
        # epilogue on the GPU's own output: next input within one bf16 ulp
        r, x_next = mo.stack_epilogue(r, got["y_all"][l].astype(np.float64))
        if l + 1 < wl.layers:
            nxt = got["x_all"][l + 1].view(np.uint16).astype(np.int64)
            diff = np.abs(nxt - x_next.astype(np.int64))
            assert diff.max() <= 1, f"layer {l} epilogue differs by {diff.max()} bf16 ulps"
    assert_close(got["r"], r, "final residual")


@pytest.mark.parametrize("wl", [STACK, STACK8], ids=["int4", "int8"])
def test_graph_replay_matches_eager_bitwise(wl):
    import torch
    from int4_routed_expert_router_amd import api
    st = Stack(wl, 40, 0)
    st.run_eager()
    want = st.snapshot()
    stream = torch.cuda.Stream()
    g = api.StackGraph(st.desc, st.layers, st.x0, st.r, st.x_buf, st.ws, stream, **st.captures())
    for rep in range(3):
        # the program's own eager work between replays
        st.y_all.zero_()
        st.r.copy_(st.r0)
        torch.cuda.synchronize()
        g.launch(stream)
        torch.cuda.synchronize()
        got = st.snapshot()
        for k in want:
            assert np.array_equal(got[k], want[k]), f"replay {rep}: {k} differs from the eager run"
    g.close()
