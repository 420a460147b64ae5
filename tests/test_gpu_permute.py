"""Token-to-expert bucketing on the GPU: exact (integer) against a stable sort."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,E,K,skew", [(64, 512, 10, 1.3), (1, 16, 2, 0.0), (7, 24, 3, 0.0), (300, 1024, 8, 1.1),
                                        (130, 64, 64, 0.0)])
def test_permute_matches_stable_sort(T, E, K, skew):
    import torch
    from int4_routed_expert_router_amd import api
    rng = np.random.default_rng(T * 1000 + E)
    idx = np.zeros((T, K), np.int32)
    p = np.ones(E) if skew == 0 else 1.0 / np.arange(1, E + 1) ** skew
    p = p / p.sum()
    for t in range(T):
        idx[t] = rng.choice(E, size=K, replace=False, p=p)
    desc = api.Desc(256, E, K, 64, 64, 32, "bf16", 2)
    ti = torch.from_numpy(idx).cuda()
    off = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((T * K,), -7, dtype=torch.int32, device="cuda")
    inv = torch.full((T * K,), -7, dtype=torch.int32, device="cuda")
    api.permute(desc, ti, off, perm, inv)
    torch.cuda.synchronize()
    flat = idx.reshape(-1)
    want_perm = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    want_off = np.concatenate([[0], np.cumsum(counts)])
    assert np.array_equal(off.cpu().numpy(), want_off)
    assert np.array_equal(perm.cpu().numpy(), want_perm)
    want_inv = np.empty_like(want_perm)
    want_inv[want_perm] = np.arange(T * K)
    assert np.array_equal(inv.cpu().numpy(), want_inv)
