"""Generator checks: Philox known answers, determinism, value ranges."""
import os

import numpy as np

import synth
from synth.philox import philox4x32_10

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(v, 16) for v in line.split()])
    return rows


def test_philox_known_answers():
    for r in load_kat():
        out = philox4x32_10(*r[:6])
        assert [int(v) for v in out] == r[6:]


def test_expert_streams_are_independent_of_order():
    wl = synth.TINY
    a = synth.expert_raw(wl, 0, 5)
    _ = synth.expert_raw(wl, 0, 4)
    b = synth.expert_raw(wl, 0, 5)
    for k in a:
        for x, y in zip(a[k], b[k]):
            assert np.array_equal(x, y)
    c = synth.expert_raw(wl, 0, 6)
    assert not np.array_equal(a["gate"][0], c["gate"][0])
    s = synth.expert_raw(wl, 0, 0, shared=True)
    d = synth.expert_raw(wl, 0, wl.n_experts)      # shared expert has id E
    assert np.array_equal(s["down"][0], d["down"][0])


def test_value_ranges_and_bias():
    wl = synth.DEC80
    raw = synth.expert_raw(wl, 3, 77)
    q, s, b = raw["gate"]
    assert q.shape == (512, 2048) and s.shape == (512, 32)
    assert q.min() == 0 and q.max() == 15
    sv = s.view(np.float16).astype(np.float64)
    assert sv.min() >= 0.001 - 1e-6 and sv.max() <= 0.01 + 1e-5
    assert abs(sv.mean() - 0.0055) < 5e-4
    assert np.array_equal(b.view(np.float16).astype(np.float64), -8 * sv)
    counts = np.bincount(q.reshape(-1), minlength=16)
    assert counts.min() > 0.9 * q.size / 16


def test_int8_values_bytes_and_bias():
    wl = synth.DEC80I8
    raw = synth.expert_raw(wl, 3, 77)
    q, s, b = raw["gate"]
    assert q.shape == (512, 2048) and q.min() == 0 and q.max() == 255
    sv = s.view(np.float16).astype(np.float64)
    assert sv.min() >= 1e-4 - 1e-7 and sv.max() <= 1e-3 + 1e-6
    assert np.array_equal(b.view(np.float16).astype(np.float64), -128 * sv)
    # value j is byte j % 4 of word (j % 16) // 4 of Philox block j // 16
    from synth.philox import philox4x32_10
    from synth.recipes import T_GATE_Q
    words = philox4x32_10(np.uint32(2), 77, T_GATE_Q, 0, wl.weight_seed, 3)
    flat = q.reshape(-1)
    for j in range(32, 48):
        assert flat[j] == (int(words[(j % 16) // 4]) >> (8 * (j % 4))) & 0xFF


def test_router_bias_is_zipf():
    wl = synth.DEC80
    beta = synth.router_bias(wl, 0).astype(np.float64)
    p = np.exp(beta) / np.exp(beta).sum()
    ranks = np.argsort(-p)
    # the r-th most likely expert has probability proportional to r^-s
    ratio = p[ranks[0]] / p[ranks[9]]
    assert abs(ratio - 10 ** 1.1) < 1e-3 * 10 ** 1.1
    assert synth.router_bias(synth.TINY, 0) is None
    assert not np.array_equal(synth.router_bias(synth.POOL80, 0, epoch=1), synth.router_bias(synth.POOL80, 0, epoch=2))


def test_tokens_and_router_weights():
    x = synth.tokens(synth.BAT80)
    assert x.shape == (64, 2048) and x.dtype == np.uint16
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    assert abs(xf.std() - 1.0) < 0.02
    wr = synth.router_weights(synth.DEC35, 0)
    assert wr.shape == (257, 2048)
    assert abs(wr.view(np.float16).astype(np.float64).std() - 1 / np.sqrt(2048)) < 1e-3
    xt = synth.tokens(synth.TINY)
    assert xt.shape == (4, 256)


def test_bf16_rounding_of_draws():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -3.140625], np.float32)
    assert synth.f32_to_bf16_bits(v).tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC049]


def test_tiny_oracle_regression_snapshot():
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(GOLDEN, "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    out = mg.tiny_oracle()
    ref = np.load(os.path.join(GOLDEN, "tiny_layer_oracle.npz"))
    assert np.array_equal(out["idx"], ref["idx"])
    for k in ("y", "w", "gamma", "z"):
        assert np.allclose(out[k], ref[k], rtol=1e-13, atol=1e-15)


def test_gdn_inputs_shapes_and_ranges():
    wl = synth.GDN80
    q, k, v, g, beta = synth.gdn_inputs(wl, 3, 1, batch=4)
    assert q.shape == k.shape == (4, 16, 128) and v.shape == (4, 32, 128) and q.dtype == np.uint16
    assert g.shape == beta.shape == (4, 32) and g.dtype == beta.dtype == np.float32
    assert (g <= 0).all() and (np.exp(g) >= 0.85 - 1e-6).all() and ((beta >= 0) & (beta <= 1)).all()
    q2 = synth.gdn_inputs(wl, 3, 1, batch=4)[0]
    assert np.array_equal(q, q2)                          # seeded
    assert not np.array_equal(q, synth.gdn_inputs(wl, 3, 2, batch=4)[0])
    st = synth.gdn_state(synth.GDN_TINY, 0)
    assert st.shape == (3, 4, 32, 128) and st.dtype == np.float32 and 0.04 < st.std() < 0.06
