"""Inputs the kernels must survive without touching memory they do not own:
expert indices outside [0, E) (the row selects no expert and adds nothing)
and NaN router logits (selection still returns K distinct indices in range)."""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import moe_oracle as mo
from moe_testlib import DeviceLayer, assert_close, desc_for

pytestmark = pytest.mark.gpu

RAGGED = dataclasses.replace(synth.TINY, name="ragged_guard", hidden=320, n_experts=24, top_k=3, inter=192,
                             shared_inter=128, group=64, tokens=13, act_dtype="bf16", weight_seed=21,
                             token_seed=121, scale_lo=0.001, scale_hi=0.01, router_sigma=0.056, zipf_s=1.1)


@pytest.mark.parametrize("path", [1, 2], ids=["gemv", "grouped"])
def test_out_of_range_indices_add_nothing(path):
    import torch
    from int4_routed_expert_router_amd import api
    wl = RAGGED
    dl = DeviceLayer(wl, 0, use_gpu_fill=False)
    x_bits = synth.tokens(wl)
    T, K, E = wl.tokens, wl.top_k, wl.n_experts
    rng = np.random.default_rng(5)
    idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    # poison a few entries: above E, negative, far out of range
    idx[1, 0] = E
    idx[4, 2] = -1
    idx[7, 1] = E + 1000
    idx[12, 0] = -2 ** 31
    w = rng.uniform(0.1, 1.0, size=(T, K)).astype(np.float32)
    gamma = rng.uniform(0.2, 0.8, size=T).astype(np.float32)
    desc = desc_for(wl, path=path)
    x = torch.from_numpy(x_bits.view(np.int16).copy()).cuda()
    y = torch.empty(T, wl.hidden, dtype=torch.float32, device="cuda")
    ti, tw, tg = (torch.from_numpy(v).cuda() for v in (idx, w, gamma))
    api.expert_ffn(desc, dl.api_layer(), x, ti, tw, tg, y)
    torch.cuda.synchronize()
    x64 = mo.act_bits_to_f64(x_bits, wl.act_dtype)
    sh = dl.oracle_shared()
    ref = np.zeros((T, wl.hidden))
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            if 0 <= e < E:
                ex = dl.oracle_expert(e)
                ref[t] += float(w[t, k]) * mo.expert_ffn(x64[t], ex.wg, ex.wu, ex.wd)
        ref[t] += float(gamma[t]) * mo.expert_ffn(x64[t], sh.wg, sh.wu, sh.wd)
    assert_close(y.cpu().numpy(), ref, f"path {path} with dropped rows")


def test_permute_drops_out_of_range_rows():
    import torch
    from int4_routed_expert_router_amd import api
    T, K, E = 9, 4, 16
    rng = np.random.default_rng(9)
    idx = rng.integers(0, E, size=(T, K)).astype(np.int32)
    idx[0, 1] = E
    idx[3, 3] = -5
    idx[8, 0] = 1 << 30
    desc = api.Desc(256, E, K, 64, 64, 32, "bf16", 2)
    off = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((T * K,), -7, dtype=torch.int32, device="cuda")
    inv = torch.full((T * K,), -7, dtype=torch.int32, device="cuda")
    api.permute(desc, torch.from_numpy(idx).cuda(), off, perm, inv)
    torch.cuda.synchronize()
    flat = idx.reshape(-1)
    ok = (flat >= 0) & (flat < E)
    keep = np.nonzero(ok)[0]
    want_perm = keep[np.argsort(flat[keep], kind="stable")]
    want_off = np.concatenate([[0], np.cumsum(np.bincount(flat[keep], minlength=E))])
    n_ok = len(keep)
    assert np.array_equal(off.cpu().numpy(), want_off)
    assert np.array_equal(perm.cpu().numpy()[:n_ok], want_perm)
    got_inv = inv.cpu().numpy()
    assert (got_inv[~ok] == -1).all()
    want_inv = np.empty(T * K, np.int64)
    want_inv[want_perm] = np.arange(n_ok)
    assert np.array_equal(got_inv[ok], want_inv[ok])


def test_nan_logits_still_select_valid_experts():
    import torch
    from int4_routed_expert_router_amd import api
    wl = RAGGED
    dl = DeviceLayer(wl, 0, use_gpu_fill=False)
    x_bits = synth.tokens(wl).copy()
    nan = 0x7FC0
    x_bits[2, :] = nan          # every logit of token 2 is NaN
    x_bits[5, 17] = nan         # one NaN column poisons token 5 too
    T, K, E = wl.tokens, wl.top_k, wl.n_experts
    desc = desc_for(wl, path=2)
    x = torch.from_numpy(x_bits.view(np.int16).copy()).cuda()
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    g = torch.empty(T, dtype=torch.float32, device="cuda")
    y = torch.empty(T, wl.hidden, dtype=torch.float32, device="cuda")
    api.route(desc, dl.api_layer(), x, idx, w, g)
    api.layer_forward(desc, dl.api_layer(), x, y)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    assert ((got >= 0) & (got < E)).all()
    for t in range(T):
        assert len(set(got[t].tolist())) == K
    # tokens without NaN are unaffected: finite outputs
    yy = y.cpu().numpy()
    clean = [t for t in range(T) if t not in (2, 5)]
    assert np.isfinite(yy[clean]).all()
