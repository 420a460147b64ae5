"""Top-K selection under heavy ties, at every per-lane depth of the kernel.

Router rows and activations take values in {-1, 0, 1}, so every logit is a
small integer that any summation order reproduces exactly: the kernel's
logits must equal the integer dot products bit for bit, and its selection
must equal the oracle's (value desc, expert index asc) order on them.  With
at most 2H+1 distinct logits over up to 1000 experts, ties inside one lane's
list and across lanes occur on nearly every token.  A bias of -inf on some
experts exercises the bottom of the order (K = E selects them all)."""
import numpy as np
import pytest

from oracle import moe_oracle as mo

pytestmark = pytest.mark.gpu

# (E, K, T, H): per-lane depths 1, 2, 4, 8 and 16; E = 100 leaves the last
# lane entries partly empty; T = 70 spans several top-k workgroups.  From 16
# tokens the router runs on the matrix cores over hidden-dimension slices:
# 2 slices at (256, 70, 64) and (512, 64, 128), 4 at (512, 16, 256).
CASES = [(20, 20, 7, 64), (100, 10, 9, 128), (256, 8, 70, 64), (512, 10, 64, 128), (512, 10, 16, 256),
         (1000, 64, 5, 64)]

F16_BITS = {-1: 0xBC00, 0: 0x0000, 1: 0x3C00}
BF16_BITS = {-1: 0xBF80, 0: 0x0000, 1: 0x3F80}


def _bits(v, table):
    out = np.zeros(v.shape, dtype=np.uint16)
    for k, b in table.items():
        out[v == k] = b
    return out


@pytest.mark.parametrize("E,K,T,H", CASES, ids=[f"E{c[0]}_K{c[1]}_T{c[2]}" for c in CASES])
def test_topk_exact_ties(E, K, T, H):
    import torch
    from int4_routed_expert_router_amd import api
    rng = np.random.default_rng(E * 7 + K)
    w_int = rng.integers(-1, 2, size=(E + 1, H))
    x_int = rng.integers(-1, 2, size=(T, H))
    bias = np.zeros(E, dtype=np.float32)
    if E == 20:
        bias[[3, 4, 11, 17, 19]] = -np.inf
    desc = api.Desc(hidden=H, n_experts=E, top_k=K, inter=64, shared_inter=0, group_size=64, act_dtype="bf16")
    stride = -(-desc.blob_bytes // 256) * 256
    dummy = torch.zeros(256, dtype=torch.uint8, device="cuda")   # expert blobs are not read by routing
    rw = torch.from_numpy(_bits(w_int, F16_BITS).view(np.int16).copy()).cuda()
    rb = torch.from_numpy(bias).cuda()
    layer = api.Layer(rw, rb, dummy, stride)
    x = torch.from_numpy(_bits(x_int, BF16_BITS).view(np.int16).copy()).cuda()
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, K, dtype=torch.float32, device="cuda")
    gam = torch.empty(T, dtype=torch.float32, device="cuda")
    logits = torch.empty(T, E + 1, dtype=torch.float32, device="cuda")
    api.route(desc, layer, x, idx, wt, gam, logits)
    torch.cuda.synchronize()
    z_exact = (x_int @ w_int.T).astype(np.float64)
    z_exact[:, :E] += bias
    z = logits.cpu().numpy().astype(np.float64)
    bad = np.argwhere(~(z == z_exact))
    assert len(bad) == 0, f"integer logits must be exact: {len(bad)} differ, first (token, row) {bad[:4].tolist()}"
    got_i, got_w, got_g = idx.cpu().numpy(), wt.cpu().numpy(), gam.cpu().numpy()
    n_tied = 0
    for t in range(T):
        want = mo.topk_order(z_exact[t, :E], K)
        assert got_i[t].tolist() == want.tolist(), f"token {t}"
        n_tied += len(np.unique(z_exact[t, want])) < K
        np.testing.assert_allclose(got_w[t], mo.renormalised_weights(z_exact[t, want]), rtol=2e-6, atol=1e-7)
        np.testing.assert_allclose(got_g[t], mo.sigmoid(z_exact[t, E]), rtol=2e-6, atol=1e-7)
    assert n_tied > 0, "the case must contain ties inside the selection"
