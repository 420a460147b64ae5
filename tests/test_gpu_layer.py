"""GPU parity of the MoE block against the fp64 oracle (through the C ABI)."""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import moe_oracle as mo
from moe_testlib import DeviceLayer, act_to_f64, assert_close, check_routing, desc_for

pytestmark = pytest.mark.gpu

RAGGED = dataclasses.replace(synth.TINY, name="ragged", hidden=320, n_experts=24, top_k=3, inter=192,
                             shared_inter=128, group=64, tokens=7, act_dtype="bf16", weight_seed=11, token_seed=111,
                             scale_lo=0.001, scale_hi=0.01, router_sigma=0.056, zipf_s=1.1)
TINY_KE = dataclasses.replace(synth.TINY, name="tiny_k_eq_e", top_k=16, weight_seed=12, token_seed=112)
TINY_G128 = dataclasses.replace(synth.TINY, name="tiny_g128", inter=128, shared_inter=128, group=128,
                                act_dtype="bf16", weight_seed=13, token_seed=113)


def run_layer(wl, dl, x_bits, path, shared=True):
    import torch
    from int4_routed_expert_router_amd import api
    desc = desc_for(wl, path=path, shared_inter=None if shared else 0)
    T = x_bits.shape[0]
    x = torch.from_numpy(x_bits.view(np.int16).copy()).cuda()
    y = torch.empty(T, wl.hidden, dtype=torch.float32, device="cuda")
    idx = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda")
    g = torch.empty(T, dtype=torch.float32, device="cuda")
    logits = torch.empty(T, wl.n_experts + 1, dtype=torch.float32, device="cuda")
    ws = api.workspace(desc, T)
    layer = dl.api_layer()
    api.route(desc, layer, x, idx, w, g, logits, ws=ws)
    api.layer_forward(desc, layer, x, y, ws=ws)
    torch.cuda.synchronize()
    return dict(y=y.cpu().numpy(), idx=idx.cpu().numpy(), w=w.cpu().numpy(), gamma=g.cpu().numpy(),
                logits=logits.cpu().numpy())


def oracle_layer(wl, dl, x_bits, gpu, shared=True):
    x64 = mo.act_bits_to_f64(x_bits, wl.act_dtype)
    wr64 = dl.router_f64()
    b64 = dl.bias_f64()
    sets, flagged = check_routing(gpu["idx"], gpu["w"], gpu["logits"], x64, wr64, b64, wl.top_k)
    out = mo.layer_forward(x64, wr64, b64, dl.oracle_expert, dl.oracle_shared() if shared else None, wl.top_k,
                           forced_idx=sets)
    return out, flagged


def check_layer(wl, path, layer=0, general_bias_seed=None, shared=True, gpu_fill=True, x_bits=None):
    dl = DeviceLayer(wl, layer, use_gpu_fill=gpu_fill, general_bias_seed=general_bias_seed)
    if x_bits is None:
        x_bits = synth.tokens(wl)
    gpu = run_layer(wl, dl, x_bits, path, shared)
    ref, flagged = oracle_layer(wl, dl, x_bits, gpu, shared)
    assert_close(gpu["logits"][:, :-1], ref["z"], "logits")
    assert_close(gpu["w"], ref["w"], "routing weights")
    if shared:
        assert_close(gpu["gamma"], ref["gamma"], "shared gate")
    worst, tol = assert_close(gpu["y"], ref["y"], f"{wl.name} layer output")
    assert np.isfinite(gpu["y"]).all()
    return worst, tol, flagged


@pytest.mark.parametrize("path", [1, 2], ids=["gemv", "grouped"])
def test_tiny_layer(path):
    check_layer(synth.TINY, path, gpu_fill=False)


@pytest.mark.parametrize("path", [1, 2], ids=["gemv", "grouped"])
def test_ragged_layer(path):
    check_layer(RAGGED, path, gpu_fill=False)


@pytest.mark.parametrize("path", [1, 2], ids=["gemv", "grouped"])
def test_general_affine_bias(path):
    check_layer(RAGGED, path, general_bias_seed=5)


@pytest.mark.parametrize("path", [1, 2], ids=["gemv", "grouped"])
def test_no_shared_expert(path):
    check_layer(synth.TINY, path, shared=False, gpu_fill=False)


@pytest.mark.parametrize("path", [1, 2], ids=["gemv", "grouped"])
def test_k_equals_e(path):
    check_layer(TINY_KE, path, gpu_fill=False)


@pytest.mark.parametrize("path", [1, 2], ids=["gemv", "grouped"])
def test_group_128(path):
    check_layer(TINY_G128, path, gpu_fill=False)


def test_gpu_fill_matches_host_packer():
    import torch
    from int4_routed_expert_router_amd import api
    for wl, experts in ((synth.TINY, [0, 7, 15]), (synth.DEC80, [0, 311]), (RAGGED, [23])):
        stride = api.blob_bytes(wl.hidden, wl.inter, wl.group)
        dev = torch.empty(stride * len(experts), dtype=torch.uint8, device="cuda")
        for k, e in enumerate(experts):
            api.synth_fill_experts(wl.weight_seed, 3, e, 1, wl.hidden, wl.inter, wl.group, wl.scale_lo, wl.scale_hi,
                                   dev[k * stride:], stride)
        got = dev.cpu().numpy()
        for k, e in enumerate(experts):
            raw = synth.expert_raw(wl, 3, e)
            want = api.pack_expert(raw, wl.hidden, wl.inter, wl.group)
            assert np.array_equal(got[k * stride:(k + 1) * stride], want), (wl.name, e)


def test_gpu_philox_known_answers():
    import torch
    from int4_routed_expert_router_amd import api
    from test_synth import load_kat
    rows = np.array(load_kat(), dtype=np.uint64).astype(np.uint32)
    ctr = torch.from_numpy(rows[:, :4].astype(np.int64).astype(np.int32)).cuda()
    key = torch.from_numpy(rows[:, 4:6].astype(np.int64).astype(np.int32)).cuda()
    out = torch.zeros(len(rows), 4, dtype=torch.int32, device="cuda")
    api.synth_philox(ctr, key, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), rows[:, 6:10])


@pytest.mark.parametrize("wl_name,layer", [("dec35", 0), ("dec80", 0), ("dec80", 47)])
def test_decode_layer_full_size(wl_name, layer):
    wl = synth.WORKLOADS[wl_name]
    worst, tol, flagged = check_layer(wl, 0, layer=layer)
    print(f"{wl_name} layer {layer}: max err {worst:.3e} (tol {tol:.3e}), near ties {flagged}")


@pytest.mark.parametrize("path", [1, 2], ids=["gemv", "grouped"])
def test_batched_layer_full_size(path):
    wl = synth.BAT80
    worst, tol, flagged = check_layer(wl, path, layer=5)
    print(f"bat80 path {path}: max err {worst:.3e} (tol {tol:.3e}), near ties {flagged}")


@pytest.mark.parametrize("n_tokens", [17, 128])
def test_batched_layer_full_size_other_batches(n_tokens):
    # the full 2048/512 shape (the shape-specialised grouped kernels) at other
    # batch sizes: 17 tokens leave a one-row shared unit and mostly one-row
    # experts, 128 tokens give hot experts up to eight units
    wl = synth.BAT80
    x_bits = synth.tokens(wl, n_tokens=n_tokens, seed=wl.token_seed + n_tokens)
    worst, tol, flagged = check_layer(wl, 2, layer=11, x_bits=x_bits)
    print(f"bat80 shape, {n_tokens} tokens, grouped: max err {worst:.3e} (tol {tol:.3e}), near ties {flagged}")


def test_grouped_ranges_over_many_units():
    # 4096 tokens of the tiny layer: 775 units of 16 rows, so every grouped
    # workgroup's range crosses several units (about 12 gate/up pair-tiles of
    # 4 per unit, about 6 down quads of 2 per unit: the down kernel restages h
    # into a buffer it used two units before)
    wl = dataclasses.replace(synth.TINY, name="tiny_t4096", tokens=4096, token_seed=114)
    worst, tol, flagged = check_layer(wl, 2)
    print(f"tiny, 4096 tokens, grouped: max err {worst:.3e} (tol {tol:.3e}), near ties {flagged}")


def test_exact_ties_pick_lower_index():
    import torch
    from int4_routed_expert_router_amd import api
    wl = dataclasses.replace(synth.TINY, name="ties", act_dtype="bf16")
    # expert 9 duplicates expert 3's router row; with x = 0 only the bias decides
    dl = DeviceLayer(wl, 0, use_gpu_fill=False, dup_rows=[(9, 3), (12, 3)])
    desc = desc_for(wl)
    T = 3
    x_bits = synth.tokens(wl, T)
    x_bits[2] = 0
    x = torch.from_numpy(x_bits.view(np.int16).copy()).cuda()
    idx = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda")
    logits = torch.empty(T, wl.n_experts + 1, dtype=torch.float32, device="cuda")
    api.route(desc, dl.api_layer(), x, idx, w, None, logits)
    torch.cuda.synchronize()
    z = logits.cpu().numpy()
    for t in range(T):
        assert z[t, 3] == z[t, 9] == z[t, 12]
        assert idx.cpu().numpy()[t].tolist() == mo.topk_order(z[t, :-1].astype(np.float64), wl.top_k).tolist()
    # x = 0: every logit is 0 (no bias in this workload) -> experts 0 and 1 with w = 1/2
    assert idx.cpu().numpy()[2].tolist() == [0, 1]
    assert np.all(w.cpu().numpy()[2] == 0.5)


def test_zero_tokens_is_noop():
    import torch
    from int4_routed_expert_router_amd import api
    wl = synth.TINY
    dl = DeviceLayer(wl, 0, use_gpu_fill=False)
    desc = desc_for(wl)
    x = torch.zeros(0, wl.hidden, dtype=torch.int16, device="cuda")
    y = torch.zeros(0, wl.hidden, dtype=torch.float32, device="cuda")
    api.layer_forward(desc, dl.api_layer(), x, y, ws=torch.empty(256, dtype=torch.uint8, device="cuda"))


def test_path_cross_check():
    """GEMV family vs grouped family on the same batch: same routing, outputs
    within the oracle tolerance of each other."""
    wl = RAGGED
    dl = DeviceLayer(wl, 0, use_gpu_fill=False)
    x_bits = synth.tokens(wl)
    a = run_layer(wl, dl, x_bits, 1)
    b = run_layer(wl, dl, x_bits, 2)
    assert np.array_equal(a["idx"], b["idx"])
    assert_close(b["y"], a["y"], "grouped vs GEMV")


def test_deterministic_repeat():
    wl = RAGGED
    dl = DeviceLayer(wl, 0, use_gpu_fill=False)
    x_bits = synth.tokens(wl)
    for path in (1, 2):
        a = run_layer(wl, dl, x_bits, path)
        b = run_layer(wl, dl, x_bits, path)
        assert np.array_equal(a["y"], b["y"])


def fused_and_separate(wl, dl, x_bits):
    """One layer call with the selection inside the gate/up kernel, then
    moe_route + moe_expert_ffn (the top-K kernel); returns both results as
    [y, idx, w, gamma] and the router logits of the separate call."""
    import torch
    from int4_routed_expert_router_amd import api
    desc = desc_for(wl, path=1)
    x = torch.from_numpy(x_bits.view(np.int16).copy()).cuda()
    T, K, H = x_bits.shape[0], wl.top_k, wl.hidden
    layer = dl.api_layer()
    ws = api.workspace(desc, T)
    outs = []
    logits = torch.full((T, wl.n_experts + 1), float("nan"), dtype=torch.float32, device="cuda")
    for fused in (True, False):
        y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
        w = torch.full((T, K), float("nan"), dtype=torch.float32, device="cuda")
        g = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
        if fused:
            api.layer_forward(desc, layer, x, y, idx, w, g, ws=ws)
        else:
            api.route(desc, layer, x, idx, w, g, logits, ws=ws)
            api.expert_ffn(desc, layer, x, idx, w, g, y, ws=ws)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (y, idx, w, g)])
    return outs, logits.cpu().numpy()


WIDE_K32 = dataclasses.replace(synth.DEC80, name="wide_k32", hidden=256, inter=128, shared_inter=128, top_k=32,
                               weight_seed=14, token_seed=114)


@pytest.mark.parametrize("wl,n_tokens", [(synth.TINY, 4), (RAGGED, 7), (synth.DEC80, 1), (synth.DEC80, 3),
                                         (WIDE_K32, 1)],
                         ids=["tiny_E16", "ragged_E24", "dec80_T1", "dec80_T3", "E512_K32_T1"])
def test_fused_topk_gemv_matches_separate_kernels(wl, n_tokens):
    """On the GEMV family a layer call selects the experts inside the gate/up
    kernel (no top-K launch); moe_route + moe_expert_ffn run the top-K
    kernel.  Same code, same order: bit-identical selection, weights, gate
    and output."""
    dl = DeviceLayer(wl, 2)
    outs, _ = fused_and_separate(wl, dl, synth.tokens(wl, n_tokens=n_tokens))
    for name, a, b in zip(("y", "idx", "w", "gamma"), outs[0], outs[1]):
        assert np.array_equal(a, b), f"{wl.name} T={n_tokens}: {name} differs between fused and separate top-K"
    assert np.isfinite(outs[0][0]).all()


@pytest.mark.parametrize("base,tied", [
    (synth.DEC80, [5, 6, 69, 70, 133, 197, 300, 301, 511]),   # lanes 5, 6, 5, 6, 5, 5, 44, 45, 63
    (synth.DEC35, [5, 6, 69, 70, 133, 197, 255]),             # lanes 5, 6, 5, 6, 5, 5, 63
], ids=["dec80", "dec35"])
def test_fused_topk_gemv_exact_ties(base, tied):
    """Experts with the same router row (no bias) tie for the top of the
    token's selection, across lanes and within a lane's list of the wave
    selection (expert e sits in lane e % 64).  Inside the gate/up kernel a
    workgroup of rank k runs only the first k + 1 selection rounds; every
    rank must still get the expert of the whole selection (ties to the lower
    expert index), bit for bit as the top-K kernel gives it."""
    import torch
    wl = dataclasses.replace(base, name=base.name + "_ties", zipf_s=0.0)
    assert len(tied) < wl.top_k
    x_bits = synth.tokens(wl, 1)
    xf = (x_bits.astype(np.uint32) << 16).view(np.float32)[0]
    row = synth.f32_to_f16_bits(np.where(xf >= 0, 0.02, -0.02).astype(np.float32))
    dl = DeviceLayer(wl, 0)
    for e in tied:
        dl.router_bits[e] = row
    dl.router_w.copy_(torch.from_numpy(dl.router_bits.view(np.int16).copy()))
    outs, z = fused_and_separate(wl, dl, x_bits)
    for name, a, b in zip(("y", "idx", "w", "gamma"), outs[0], outs[1]):
        assert np.array_equal(a, b), f"{name} differs between fused and separate top-K"
    assert len(set(z[0, tied].tolist())) == 1 and z[0, tied[0]] > np.delete(z[0, :-1], tied).max()
    idx = outs[0][1][0]
    assert idx[:len(tied)].tolist() == tied
    assert idx.tolist() == mo.topk_order(z[0, :-1].astype(np.float64), wl.top_k).tolist()
    assert np.isfinite(outs[0][0]).all()
