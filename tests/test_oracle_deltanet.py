"""Pins of the Gated DeltaNet oracle against what the gated delta rule fixes:
closed forms of special cases, several steps against the whole-sequence
matrix-product form, the key-head grouping and the normalisation."""
import numpy as np

from oracle import deltanet_oracle as dn


def _rand(seed, B=2, Hk=2, Hv=4, dk=16, dv=8):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hv, dv, dk)), rng.standard_normal((B, Hk, dk)),
            rng.standard_normal((B, Hk, dk)), rng.standard_normal((B, Hv, dv)),
            -rng.uniform(0.0, 0.5, (B, Hv)), rng.uniform(0.0, 1.0, (B, Hv)))


def test_beta_zero_only_decays():
    S, q, k, v, g, _ = _rand(1)
    new, o = dn.gdn_step(S, q, k, v, g, np.zeros_like(g), 0.5)
    a = np.exp(g)[..., None, None]
    assert np.allclose(new, a * S, rtol=0, atol=1e-14)
    qn = np.repeat(q / np.linalg.norm(q, axis=-1, keepdims=True), 2, axis=1) * 0.5
    assert np.allclose(o, np.einsum("bhij,bhj->bhi", a * S, qn), rtol=1e-6, atol=1e-9)


def test_delta_rule_writes_v_at_k():
    # alpha = 1, beta = 1: the new state maps k^ exactly to v
    S, q, k, v, g, _ = _rand(2)
    new, _ = dn.gdn_step(S, q, k, v, np.zeros_like(g), np.ones_like(g), 1.0)
    kn = np.repeat(dn.l2_normalise(k), 2, axis=1)
    # |k^| = |k| / sqrt(|k|^2 + eps), so S' k^ = v + (1 - |k^|^2) (S k^ - v) exactly
    n2 = (kn * kn).sum(-1, keepdims=True)
    sk = np.einsum("bhij,bhj->bhi", S, kn)
    want = v + (1.0 - n2) * (sk - v)
    assert np.allclose(np.einsum("bhij,bhj->bhi", new, kn), want, rtol=0, atol=1e-12)
    assert np.abs(np.einsum("bhij,bhj->bhi", new, kn) - v).max() < 1e-5


def test_zero_state_is_rank_one_write():
    S, q, k, v, g, beta = _rand(3)
    new, o = dn.gdn_step(np.zeros_like(S), q, k, v, g, beta, 2.0)
    kn = np.repeat(dn.l2_normalise(k), 2, axis=1)
    qn = np.repeat(dn.l2_normalise(q), 2, axis=1) * 2.0
    assert np.allclose(new, beta[..., None, None] * v[..., :, None] * kn[..., None, :], rtol=0, atol=1e-14)
    kq = (kn * qn).sum(-1)
    assert np.allclose(o, (beta * kq)[..., None] * v, rtol=0, atol=1e-12)


def test_steps_equal_whole_sequence_form():
    # S_T = S_0 M_1 ... M_T + sum_t beta_t v_t k_t^T M_{t+1} ... M_T with
    # M_t = alpha_t (I - beta_t k_t k_t^T): the definition's matrix products,
    # one head at a time, against the oracle stepped T times
    rng = np.random.default_rng(4)
    B, Hk, Hv, dk, dv, T = 1, 1, 2, 6, 5, 5
    S0 = rng.standard_normal((B, Hv, dv, dk))
    steps = [(rng.standard_normal((B, Hk, dk)), rng.standard_normal((B, Hk, dk)), rng.standard_normal((B, Hv, dv)),
              -rng.uniform(0, 1, (B, Hv)), rng.uniform(0, 1, (B, Hv))) for _ in range(T)]
    S = S0
    outs = []
    for q, k, v, g, beta in steps:
        S, o = dn.gdn_step(S, q, k, v, g, beta, 0.7)
        outs.append(o)
    for h in range(Hv):
        M = []
        for q, k, v, g, beta in steps:
            kn = k[0, 0] / np.sqrt(k[0, 0] @ k[0, 0] + dn.EPS)
            M.append(np.exp(g[0, h]) * (np.eye(dk) - beta[0, h] * np.outer(kn, kn)))
        for t in range(1, T + 1):
            St = S0[0, h].copy()
            for m in M[:t]:
                St = St @ m
            for s in range(t):
                q, k, v, g, beta = steps[s]
                kn = k[0, 0] / np.sqrt(k[0, 0] @ k[0, 0] + dn.EPS)
                term = beta[0, h] * np.outer(v[0, h], kn)
                for m in M[s + 1:t]:
                    term = term @ m
                St = St + term
            q = steps[t - 1][0][0, 0]
            qn = 0.7 * q / np.sqrt(q @ q + dn.EPS)
            assert np.allclose(St @ qn, outs[t - 1][0, h], rtol=1e-10, atol=1e-12), (h, t)
        assert np.allclose(St, S[0, h], rtol=1e-10, atol=1e-12)


def test_value_heads_share_key_heads_in_groups():
    S, q, k, v, g, beta = _rand(5, Hk=2, Hv=4)
    k = k.copy()
    k[:, 1] = 0.0            # key head 1 (value heads 2, 3) writes nothing
    new, _ = dn.gdn_step(S, q, k, v, g, beta, 1.0)
    a = np.exp(g)[..., None, None]
    assert np.allclose(new[:, 2:], a[:, 2:] * S[:, 2:], rtol=0, atol=1e-14)
    assert not np.allclose(new[:, :2], a[:, :2] * S[:, :2])


def test_rescaling_q_and_k_changes_nothing():
    S, q, k, v, g, beta = _rand(6)
    a = dn.gdn_step(S, q, k, v, g, beta, 1.0)
    b = dn.gdn_step(S, 3.0 * q, 0.25 * k, v, g, beta, 1.0)
    # only eps = 1e-6 inside the square root tells the scales apart
    for x, y in zip(a, b):
        assert np.abs(x - y).max() <= 1e-5 * np.abs(x).max()
    # (k, v) -> (-k, -v): the decay term keeps k^ k^T and the write keeps v k^T
    c = dn.gdn_step(S, q, -k, -v, g, beta, 1.0)
    assert np.allclose(c[0], a[0], rtol=0, atol=1e-12) and np.allclose(c[1], a[1], rtol=0, atol=1e-12)
