"""moe_layer_forward_static (workspace in the library's static device array,
no allocation) gives the same results as moe_layer_forward with a caller
workspace, bit for bit, on consecutive calls of decreasing size (the second
call finds the array holding the first call's contents), on both kernel
families; a batch whose workspace exceeds the array is refused."""
import numpy as np
import pytest

import synth
from moe_testlib import DeviceLayer, desc_for

pytestmark = pytest.mark.gpu


def test_static_scratch_call_equals_workspace_call():
    import torch
    from int4_routed_expert_router_amd import api, MoeError
    from int4_routed_expert_router_amd._lib import lib
    wl = synth.BAT80
    dl = DeviceLayer(wl, 3)
    desc = desc_for(wl)
    K, H = wl.top_k, wl.hidden
    x_all = torch.from_numpy(synth.tokens(wl, n_tokens=64, seed=wl.token_seed + 7).view(np.int16).copy()).cuda()
    for T in (64, 24, 2):                     # grouped, grouped (smaller), GEMV family
        x = x_all[:T].contiguous()
        outs = []
        for static in (True, False):
            y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
            idx = torch.full((T, K), -1, dtype=torch.int32, device="cuda")
            w = torch.full((T, K), float("nan"), dtype=torch.float32, device="cuda")
            g = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
            if static:
                api.layer_forward_static(desc, dl.api_layer(), x, y, idx, w, g)
            else:
                api.layer_forward(desc, dl.api_layer(), x, y, idx, w, g, ws=api.workspace(desc, T))
            torch.cuda.synchronize()
            outs.append([t.cpu().numpy() for t in (y, idx, w, g)])
        for name, a, b in zip(("y", "idx", "w", "gamma"), *outs):
            assert np.array_equal(a, b), f"T={T}: {name} differs between the static-scratch and workspace calls"
        assert np.isfinite(outs[0][0]).all()
    cap = 32 << 20
    big = 512
    assert api.workspace_bytes(desc, big) > cap
    xb = torch.zeros(big, H, dtype=torch.int16, device="cuda")
    yb = torch.empty(big, H, dtype=torch.float32, device="cuda")
    with pytest.raises(MoeError, match="MOE_EWORKSPACE"):
        api.layer_forward_static(desc, dl.api_layer(), xb, yb)
    assert b"static scratch" in lib().moe_last_error()
