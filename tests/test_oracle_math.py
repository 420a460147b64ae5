"""Pins of the fp64 oracle's arithmetic against closed forms, brute force and
invariants that do not come from the oracle itself."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import moe_oracle as mo

# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------


def test_bf16_rne_closed_forms():
    # bfloat16 keeps 8 significant bits: 1 + 2**-7 is the successor of 1.
    cases = {
        1.0: 0x3F80,
        -2.0: 0xC000,
        1.0 + 2.0 ** -7: 0x3F81,
        1.0 + 2.0 ** -8: 0x3F80,                 # halfway, ties to even (down)
        1.0 + 3 * 2.0 ** -8: 0x3F82,             # halfway, ties to even (up)
        1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F81,    # just above halfway
        0.0: 0x0000,
        3.140625: 0x4049,                        # 1.5703125 * 2: exactly representable
    }
    for v, bits in cases.items():
        assert int(mo.f64_to_bf16_bits_rne(np.array([v]))[0]) == bits, v
    # decode back
    assert mo.bf16_bits_to_f64(np.array([0x3F81], np.uint16))[0] == 1.0 + 2.0 ** -7
    assert mo.f16_bits_to_f64(np.array([0x3C00, 0xC800, 0x0001], np.uint16)).tolist() == [1.0, -8.0, 2.0 ** -24]


def test_bf16_rne_matches_exhaustive_neighbours():
    # For random doubles, the result must be one of the two bf16 neighbours and
    # the nearer one (even mantissa on exact ties).
    rng = np.random.default_rng(5)
    v = rng.standard_normal(2000) * np.exp2(rng.integers(-20, 20, 2000))
    bits = mo.f64_to_bf16_bits_rne(v)
    r = mo.bf16_bits_to_f64(bits)
    for vi, ri, bi in zip(v, r, bits):
        up = mo.bf16_bits_to_f64(np.array([bi + 1], np.uint16))[0]
        dn = mo.bf16_bits_to_f64(np.array([bi - 1], np.uint16))[0]
        assert abs(vi - ri) <= abs(vi - up) and abs(vi - ri) <= abs(vi - dn)


# ---------------------------------------------------------------------------
# affine int4 dequant
# ---------------------------------------------------------------------------


def _f16(v):
    return np.float16(v).view(np.uint16)


def test_dequant_closed_form_exact():
    rng = np.random.default_rng(1)
    rows, cols, g = 4, 64, 32
    q = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
    s = rng.uniform(0.001, 0.01, (rows, cols // g)).astype(np.float16)
    b = (s * np.float16(-8)).astype(np.float16)
    w = mo.dequant(q, s.view(np.uint16), b.view(np.uint16), g)
    for r in range(rows):
        for c in range(cols):
            exact = Fraction(float(s[r, c // g])) * (int(q[r, c]) - 8)
            assert Fraction(float(w[r, c])) == exact
            # s*(q-8) has at most 15 significant bits: exact in binary32 too
            assert float(np.float32(w[r, c])) == float(w[r, c])


def test_dequant_general_affine_and_q8_zero():
    q = np.full((2, 64), 8, np.uint8)
    s = np.array([[0.5, 0.25], [1.0, 2.0]], np.float16)
    w = mo.dequant(q, s.view(np.uint16), (s * np.float16(-8)).astype(np.float16).view(np.uint16), 32)
    assert np.all(w == 0.0)
    q2 = np.arange(128).reshape(2, 64) % 16
    b = np.array([[0.125, -3.0], [7.5, -0.0625]], np.float16)
    w2 = mo.dequant(q2, s.view(np.uint16), b.view(np.uint16), 32)
    assert w2[0, 5] == 0.5 * 5 + 0.125
    assert w2[0, 40] == 0.25 * (40 % 16) - 3.0
    assert w2[1, 63] == 2.0 * (127 % 16) - 0.0625


# ---------------------------------------------------------------------------
# top-k, weights, gate
# ---------------------------------------------------------------------------


def _brute_topk(z, k):
    return sorted(range(len(z)), key=lambda e: (-z[e], e))[:k]


def test_dequant_int8_closed_forms():
    # int8 affine: W = s*q + b with q in 0..255; b = -128 s centres the range.
    # s = 2^-8: q = 255 -> 127/256, q = 0 -> -1/2, q = 128 -> 0 (all exact in fp16 and fp64)
    s = np.full((1, 1), 0x1C00, np.uint16)      # fp16 2^-8
    b = np.full((1, 1), 0xB800, np.uint16)      # fp16 -0.5
    q = np.array([[255, 0, 128, 1] * 8], np.uint8)
    w = mo.dequant(q, s, b, 32, bits=8)
    assert w[0, 0] == 127 / 256 and w[0, 1] == -0.5 and w[0, 2] == 0.0 and w[0, 3] == -127 / 256
    with pytest.raises(ValueError):
        mo.dequant(q, s, b, 32)               # bits = 4 rejects values above 15
    with pytest.raises(ValueError):
        mo.dequant(q, s, b, 32, bits=6)


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(2)
    for _ in range(400):
        n_e = int(rng.integers(1, 14))
        k = int(rng.integers(1, n_e + 1))
        z = rng.integers(-3, 4, n_e).astype(np.float64)   # many exact ties
        assert mo.topk_order(z, k).tolist() == _brute_topk(z.tolist(), k)


def test_topk_exhaustive_small():
    # every assignment of values {0,1,2} to 5 experts, every k
    for vals in itertools.product([0.0, 1.0, 2.0], repeat=5):
        for k in range(1, 6):
            assert mo.topk_order(np.array(vals), k).tolist() == _brute_topk(list(vals), k)


def test_topk_k_equals_e_is_full_order():
    z = np.array([0.5, -1.0, 0.5, 3.0])
    assert mo.topk_order(z, 4).tolist() == [3, 0, 2, 1]


def test_weights_invariants():
    rng = np.random.default_rng(3)
    for _ in range(100):
        z = rng.standard_normal(int(rng.integers(1, 12))) * 4
        w = mo.renormalised_weights(z)
        assert abs(w.sum() - 1.0) < 1e-15
        assert np.all(w > 0)
    assert np.allclose(mo.renormalised_weights(np.full(5, 0.7)), 0.2, rtol=0, atol=1e-16)


def test_weights_softmax_closed_form_when_k_is_e():
    z = [0.3, -1.2, 2.5, 0.0]
    denom = sum(math.exp(v) for v in z)
    expect = [math.exp(v) / denom for v in z]
    idx = mo.topk_order(np.array(z), 4)
    w = mo.renormalised_weights(np.array(z)[idx])
    assert np.allclose(w, np.array(expect)[idx], rtol=1e-15, atol=0)


def test_softmax_then_renormalise_equals_restricted_softmax():
    # softmax over all E then renormalise over S == softmax over S
    rng = np.random.default_rng(4)
    z = rng.standard_normal(9)
    p = [math.exp(v) for v in z]
    tot = sum(p)
    p = [v / tot for v in p]
    idx = mo.topk_order(z, 3)
    sel = [p[i] for i in idx]
    expect = [v / sum(sel) for v in sel]
    assert np.allclose(mo.renormalised_weights(z[idx]), expect, rtol=1e-14, atol=0)


def test_sigmoid_closed_forms():
    assert mo.sigmoid(0.0) == 0.5
    assert abs(mo.sigmoid(math.log(3.0)) - 0.75) < 1e-15


def test_route_outputs_shapes_and_values():
    x = np.array([[1.0, 0.0, -1.0, 2.0]])
    wr = np.array([[1, 0, 0, 0], [0, 0, 0, 1], [0, 1, 0, 0], [0, 0, -1, 0], [0, 0, 0, 0]], np.float64)
    idx, w, gamma, z, zs = mo.route(x, wr, None, 2)
    assert z.tolist() == [[1.0, 2.0, 0.0, 1.0]]
    assert idx.tolist() == [[1, 0]]          # z0 == z3: lower index wins
    assert gamma.tolist() == [0.5]
    assert abs(w[0, 0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15


# ---------------------------------------------------------------------------
# expert FFN
# ---------------------------------------------------------------------------


def _silu_py(a):
    return a / (1.0 + math.exp(-a))


def test_expert_ffn_integer_closed_form():
    # s = 1, b = -8 gives W = q - 8: small-integer x makes a, u exact integers.
    rng = np.random.default_rng(6)
    h_dim, i_dim, g = 64, 64, 32
    one = np.full((i_dim, h_dim // g), _f16(1.0), np.uint16)
    m8 = np.full((i_dim, h_dim // g), _f16(-8.0), np.uint16)
    qg = rng.integers(0, 16, (i_dim, h_dim))
    qu = rng.integers(0, 16, (i_dim, h_dim))
    qd = rng.integers(0, 16, (h_dim, i_dim))
    wg = mo.dequant(qg, one, m8, g)
    wu = mo.dequant(qu, one, m8, g)
    wd = mo.dequant(qd, np.full((h_dim, i_dim // g), _f16(1.0), np.uint16),
                    np.full((h_dim, i_dim // g), _f16(-8.0), np.uint16), g)
    x = rng.integers(-2, 3, (1, h_dim)).astype(np.float64)
    y, a, u, h = mo.expert_ffn(x, wg, wu, wd, return_intermediates=True)
    xi = [int(v) for v in x[0]]
    for r in range(i_dim):
        a_exact = sum((int(qg[r, c]) - 8) * xi[c] for c in range(h_dim))
        u_exact = sum((int(qu[r, c]) - 8) * xi[c] for c in range(h_dim))
        assert a[0, r] == a_exact and u[0, r] == u_exact
        assert abs(h[0, r] - _silu_py(a_exact) * u_exact) <= 1e-12 * max(1.0, abs(h[0, r]))
    for n in range(h_dim):
        y_brute = sum((int(qd[n, i]) - 8) * h[0, i] for i in range(i_dim))
        assert abs(y[0, n] - y_brute) <= 1e-9 * max(1.0, abs(y_brute))


def _tiny_layer(rng, n_e=6, h_dim=64, i_dim=64, g=32, general_bias=False):
    def rand_expert():
        mats = []
        for rows, cols in ((i_dim, h_dim), (i_dim, h_dim), (h_dim, i_dim)):
            q = rng.integers(0, 16, (rows, cols))
            s = rng.uniform(0.002, 0.01, (rows, cols // g)).astype(np.float16)
            if general_bias:
                b = (-s * rng.uniform(0, 15, s.shape)).astype(np.float16)
            else:
                b = (s * np.float16(-8)).astype(np.float16)
            mats.append((q, s.view(np.uint16), b.view(np.uint16)))
        return mo.ExpertWeights.from_quant(*mats, g)

    experts = [rand_expert() for _ in range(n_e)]
    shared = rand_expert()
    wr = rng.standard_normal((n_e + 1, h_dim)) * 0.3
    bias = rng.standard_normal(n_e)
    return experts, shared, wr, bias


@pytest.mark.parametrize("general_bias", [False, True])
def test_sparse_layer_equals_dense_masked(general_bias):
    rng = np.random.default_rng(7)
    experts, shared, wr, bias = _tiny_layer(rng, general_bias=general_bias)
    x = rng.standard_normal((5, 64))
    for k in (1, 2, 6):
        sparse = mo.layer_forward(x, wr, bias, lambda e: experts[e], shared, k)
        dense = mo.layer_forward_dense(x, wr, bias, experts, shared, k)
        assert np.allclose(sparse["y"], dense, rtol=0, atol=1e-12 * np.abs(dense).max())


def test_layer_brute_force_loops():
    # pure-Python loops over the definition on a tiny layer
    rng = np.random.default_rng(8)
    experts, shared, wr, bias = _tiny_layer(rng, n_e=4)
    x = rng.standard_normal((2, 64))
    out = mo.layer_forward(x, wr, bias, lambda e: experts[e], shared, 2)
    for t in range(2):
        z = [sum(x[t, h] * wr[e, h] for h in range(64)) + bias[e] for e in range(4)]
        zs = sum(x[t, h] * wr[4, h] for h in range(64))
        sel = sorted(range(4), key=lambda e: (-z[e], e))[:2]
        ex = [math.exp(z[e] - z[sel[0]]) for e in sel]
        w = [v / sum(ex) for v in ex]
        gamma = 1.0 / (1.0 + math.exp(-zs))

        def ffn(ew):
            a = [sum(ew.wg[i, h] * x[t, h] for h in range(64)) for i in range(64)]
            u = [sum(ew.wu[i, h] * x[t, h] for h in range(64)) for i in range(64)]
            hh = [_silu_py(a[i]) * u[i] for i in range(64)]
            return [sum(ew.wd[n, i] * hh[i] for i in range(64)) for n in range(64)]

        ys = ffn(shared)
        y = [gamma * ys[n] for n in range(64)]
        for wk, e in zip(w, sel):
            ye = ffn(experts[e])
            y = [y[n] + wk * ye[n] for n in range(64)]
        assert out["idx"][t].tolist() == sel
        assert np.allclose(out["w"][t], w, rtol=1e-13, atol=0)
        assert np.allclose(out["y"][t], y, rtol=0, atol=1e-12 * max(abs(v) for v in y))


def test_zero_input_gives_zero_output():
    rng = np.random.default_rng(9)
    experts, shared, wr, bias = _tiny_layer(rng)
    out = mo.layer_forward(np.zeros((3, 64)), wr, bias, lambda e: experts[e], shared, 2)
    assert np.all(out["y"] == 0.0)
    # with x = 0 the logits are the bias alone
    assert out["idx"][0].tolist() == mo.topk_order(bias, 2).tolist()


def test_shared_only_layer():
    rng = np.random.default_rng(10)
    experts, shared, wr, bias = _tiny_layer(rng)
    zero = [mo.ExpertWeights(np.zeros((64, 64)), np.zeros((64, 64)), np.zeros((64, 64))) for _ in experts]
    x = rng.standard_normal((2, 64))
    wr[-1] = 0.0                                       # shared gate vector g = 0 -> gamma = 0.5
    out = mo.layer_forward(x, wr, bias, lambda e: zero[e], shared, 2)
    ys = mo.expert_ffn(x, shared.wg, shared.wu, shared.wd)
    assert np.all(out["gamma"] == 0.5)
    assert np.allclose(out["y"], 0.5 * ys, rtol=0, atol=1e-15)


def test_forced_index_set_renormalises_over_that_set():
    rng = np.random.default_rng(11)
    experts, shared, wr, bias = _tiny_layer(rng)
    x = rng.standard_normal((1, 64))
    out = mo.layer_forward(x, wr, bias, lambda e: experts[e], shared, 2, forced_idx=[[4, 1]])
    z = out["z"][0]
    e4, e1 = math.exp(z[4]), math.exp(z[1])
    assert np.allclose(out["w"][0], [e4 / (e4 + e1), e1 / (e4 + e1)], rtol=1e-14)


# ---------------------------------------------------------------------------
# stack epilogue and tie guard
# ---------------------------------------------------------------------------


def test_stack_epilogue_closed_form():
    r = np.zeros((1, 4))
    y = np.array([[3.0, -4.0, 0.0, 0.0]])          # mean square 25/4
    r_new, xb = mo.stack_epilogue(r, y)
    rms = math.sqrt(25.0 / 4.0 + 1e-6)
    expect = mo.f64_to_bf16_bits_rne(np.array([3.0 / rms, -4.0 / rms, 0.0, 0.0]))
    assert r_new.tolist() == [[3.0, -4.0, 0.0, 0.0]]
    assert xb[0].tolist() == expect.tolist()
    # 3/2.5 = 1.2 and 4/2.5 = 1.6 up to the eps: bf16 patterns 0x3F9A, 0xBFCD
    assert xb[0].tolist()[:2] == [0x3F9A, 0xBFCD]


def test_boundary_gap_and_error_bound():
    gap, a, b = mo.boundary_gap(np.array([1.0, 3.0, 2.5, 2.5]), 2)
    assert (gap, a, b) == (0.0, 2, 3)
    assert mo.boundary_gap(np.array([1.0, 2.0]), 2)[0] == math.inf
    x = np.array([1.0, -2.0])
    wr = np.array([[0.5, 0.25], [1.0, 1.0]])
    assert mo.logit_error_bound(x, wr, np.array([2.0]), 0) == 64 * 2.0 ** -24 * (0.5 + 0.5 + 2.0)


def test_tolerance_formula():
    assert mo.tolerance(np.array([0.5, -2.0])) == pytest.approx(2e-3 + 1e-5)
