"""GPU parity of the Gated DeltaNet step (moe_gdn_step, through the C ABI)
against the fp64 oracle: one step and chained steps, the shape edges, the
special cases of the rule, and one full 80B-shaped layer."""
import dataclasses
import math

import numpy as np
import pytest

import synth
from oracle import deltanet_oracle as dn
from oracle import moe_oracle as mo
from moe_testlib import assert_close

pytestmark = pytest.mark.gpu


def _to_dev(wl, layer, step, batch=None, state=None):
    import torch
    q, k, v, g, beta = synth.gdn_inputs(wl, layer, step, batch)
    st = synth.gdn_state(wl, layer, batch) if state is None else state
    dev = dict(q=torch.from_numpy(q.view(np.int16).copy()).cuda(), k=torch.from_numpy(k.view(np.int16).copy()).cuda(),
               v=torch.from_numpy(v.view(np.int16).copy()).cuda(), g=torch.from_numpy(g).cuda(),
               beta=torch.from_numpy(beta).cuda(), state=torch.from_numpy(st.copy()).cuda())
    host = dict(q=mo.act_bits_to_f64(q, wl.act_dtype), k=mo.act_bits_to_f64(k, wl.act_dtype),
                v=mo.act_bits_to_f64(v, wl.act_dtype), g=g.astype(np.float64), beta=beta.astype(np.float64),
                state=st.astype(np.float64))
    return dev, host


def _run(wl, dev, q_scale):
    import torch
    from int4_routed_expert_router_amd import api
    B, Hv, dv = dev["v"].shape
    o = torch.full((B, Hv, dv), float("nan"), dtype=torch.float32, device="cuda")
    api.gdn_step(dev["q"].view(B, wl.k_heads, 128), dev["k"], dev["v"], dev["g"], dev["beta"], dev["state"], o,
                 q_scale, wl.act_dtype)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def _check(wl, steps=1, q_scale=None, batch=None, edit=None):
    q_scale = 1.0 / math.sqrt(128) if q_scale is None else q_scale
    dev, host = _to_dev(wl, 0, 0, batch)
    state_ref = host["state"]
    for step in range(steps):
        if step:
            d2, h2 = _to_dev(wl, 0, step, batch, state=np.zeros(1, np.float32))
            for key in ("q", "k", "v", "g", "beta"):
                dev[key], host[key] = d2[key], h2[key]
        if edit is not None:
            edit(dev, host)
        o = _run(wl, dev, q_scale)
        state_ref, o_ref = dn.gdn_step(state_ref, host["q"], host["k"], host["v"], host["g"], host["beta"], q_scale)
        assert_close(o, o_ref, f"{wl.name} step {step} output")
        assert_close(dev["state"].cpu().numpy(), state_ref, f"{wl.name} step {step} state")
    return o


def test_tiny_one_step():
    _check(synth.GDN_TINY)


def test_tiny_chained_steps():
    _check(synth.GDN_TINY, steps=4)


@pytest.mark.parametrize("dv,hk,hv,act,b", [(16, 1, 1, "bf16", 2), (256, 2, 6, "f16", 2), (48, 3, 3, "bf16", 2),
                                            (128, 16, 32, "bf16", 1)],
                         ids=["dv16_one_head", "dv256_two_batches", "dv48_group1", "decode_batch1"])
def test_shape_edges(dv, hk, hv, act, b):
    wl = dataclasses.replace(synth.GDN_TINY, name=f"gdn_dv{dv}", head_v_dim=dv, k_heads=hk, v_heads=hv,
                             act_dtype=act, batch=b, seed=203 + dv)
    _check(wl, steps=2)


def test_beta_zero_decays_and_zero_key_writes_nothing():
    import torch
    wl = synth.GDN_TINY

    def beta0(dev, host):
        dev["beta"].zero_()
        host["beta"] = np.zeros_like(host["beta"])
    _check(wl, edit=beta0)

    def k0(dev, host):
        dev["k"].zero_()
        host["k"] = np.zeros_like(host["k"])
    _check(wl, edit=k0)
    # and with g = 0 the state is left exactly as it was when k is zero
    dev, host = _to_dev(wl, 0, 0)
    dev["k"].zero_()
    dev["g"].zero_()
    before = dev["state"].clone()
    _run(wl, dev, 0.1)
    assert torch.equal(dev["state"], before)


def test_full_size_layer():
    # 64 sequences x 32 value heads x [128 x 128] fp32 state, bf16 q, k, v
    _check(synth.GDN80, steps=2)


def test_bitwise_repeatable():
    import torch
    wl = synth.GDN_TINY
    outs = []
    for _ in range(2):
        dev, _ = _to_dev(wl, 0, 0)
        o = _run(wl, dev, 0.3)
        outs.append((o, dev["state"].cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
