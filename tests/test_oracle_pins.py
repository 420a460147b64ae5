"""Pins of two oracle functions by facts other than their own formulas.

silu: closed-form values at +-ln 3, the odd-part identity
silu(a) - silu(-a) = a, the slope 1/2 at zero, the limits for large |a|, and
the orientation of the SwiGLU product (the non-linearity is on the gate
projection, not on the up projection).

logit_error_bound: the fp32 summation orders of the two router kernels are
emulated here in numpy single precision (each fp32 addition correctly
rounded; products of a 16-bit activation and an fp16 weight are exact in
fp32), on adversarial rows (same-sign terms, heavy cancellation) and on rows
of the 80B workload's distribution.  The emulated error must stay within the
bound, the emulated trees must be no deeper than the bound's depth, and an
adversarial row must reach a quarter of the bound (so a bound much looser
than the orders' real error fails too).  The depth argument is the standard
one: a sum computed by a tree in which no term passes through more than d
roundings errs by at most d*u*sum|terms| to first order (Higham, Accuracy and
Stability of Numerical Algorithms, 2nd ed., section 4.2).

The matrix-core router step (16x16x32 products per instruction) is modelled
as a sequential fp32 sum of the instruction's 32 exact products, added to the
accumulator in one rounding: the longest chain any product can pass through
inside one instruction.
"""
import math

import numpy as np
import pytest

from oracle import moe_oracle as mo

U = 2.0 ** -24


# ---------------------------------------------------------------------------
# silu
# ---------------------------------------------------------------------------


def test_silu_closed_forms_at_ln3():
    # sigma(ln 3) = 3/4 and sigma(-ln 3) = 1/4, so silu(+-ln 3) = +-ln 3 * (3/4 or 1/4)
    ln3 = math.log(3.0)
    assert abs(float(mo.silu(ln3)) - 0.75 * ln3) <= 1e-15
    assert abs(float(mo.silu(-ln3)) + 0.25 * ln3) <= 1e-15


def test_silu_odd_part_identity():
    # a*sigma(a) - (-a)*sigma(-a) = a*(sigma(a) + sigma(-a)) = a
    a = np.linspace(-30.0, 30.0, 601)
    assert np.allclose(mo.silu(a) - mo.silu(-a), a, rtol=0, atol=1e-13)


def test_silu_slope_and_limits():
    # sigma(a) = 1/2 + a/4 - a^3/48 + a^5/480 - ..., so near zero
    # silu(a) = a/2 + a^2/4 - a^4/48 + a^6/480 + O(a^8)
    for a in (1e-4, -1e-4, 1e-6, 3e-3, -3e-3):
        assert abs(float(mo.silu(a)) - (a / 2 + a * a / 4 - a ** 4 / 48 + a ** 6 / 480)) <= 4e-16 * abs(a)
    assert float(mo.silu(0.0)) == 0.0
    # large positive: silu(a) -> a; large negative: -> 0 from below
    assert abs(float(mo.silu(40.0)) - 40.0) <= 40.0 * 1e-15
    v = float(mo.silu(-40.0))
    assert v < 0.0 and abs(v) < 1e-15
    assert abs(v + 40.0 * math.exp(-40.0)) <= 1e-30


def test_swiglu_puts_the_nonlinearity_on_the_gate():
    # one hidden unit: a = ln 3 (gate), u = 2 (up), down = 1 -> y = 2 * (3/4) ln 3
    ln3 = math.log(3.0)
    y = mo.expert_ffn(np.array([[1.0]]), np.array([[ln3]]), np.array([[2.0]]), np.array([[1.0]]))
    assert abs(float(y[0, 0]) - 1.5 * ln3) <= 1e-15
    # swapping gate and up changes the result: silu(2) * ln 3 != silu(ln 3) * 2
    y_sw = mo.expert_ffn(np.array([[1.0]]), np.array([[2.0]]), np.array([[ln3]]), np.array([[1.0]]))
    assert abs(float(y_sw[0, 0]) - 1.5 * ln3) > 0.1


# ---------------------------------------------------------------------------
# fp32 emulation of the router kernels' summation orders
# ---------------------------------------------------------------------------


class P:
    """A partial sum: fp32 value and the largest number of roundings any of
    its terms has passed through."""

    __slots__ = ("v", "d")

    def __init__(self, v, d=0):
        self.v = np.float32(v)
        self.d = d


def add(a: P, b: P) -> P:
    # both operands have at most 24 significant bits; float64 holds their sum
    # to 53 bits and the second rounding to binary32 is then innocuous
    # (53 >= 2*24 + 2), so this is the correctly rounded fp32 sum
    return P(np.float32(np.float64(a.v) + np.float64(b.v)), max(a.d, b.d) + 1)


def prod(x, w) -> P:
    # 16-bit activation (<= 11 significant bits) times fp16 weight (11 bits):
    # exact in fp32
    p = np.float64(x) * np.float64(w)
    assert np.float64(np.float32(p)) == p
    return P(p, 0)


def emu_router_vector(x, w, bias):
    """The per-row router kernel (batches below 16 tokens): lane l owns
    columns 512*it + 8*l + i and accumulates them sequentially (it, then i),
    starting from 0; the 64 lane sums are added by a butterfly over lanes in
    natural order (pairs, quads, 8s, 16s, 32s, 64); then the bias."""
    H = len(x)
    lanes = []
    for lane in range(64):
        acc = P(0.0)
        for it in range((H + 511) // 512):
            for i in range(8):
                c = 512 * it + 8 * lane + i
                if c < H:
                    acc = add(acc, prod(x[c], w[c]))
        lanes.append(acc)
    while len(lanes) > 1:
        lanes = [add(lanes[2 * j], lanes[2 * j + 1]) for j in range(len(lanes) // 2)]
    z = lanes[0]
    if bias is not None:
        z = add(z, P(np.float32(bias)))
    return z


def router_slices(H, E, T):
    """Hidden-dimension slices of the matrix-core router (as its launcher
    chooses them: double while the grid stays within 256 workgroups)."""
    tiles = ((E + 15) // 16) * ((T + 15) // 16)
    S = 1
    while S < 4 and tiles * 2 * S <= 256 and (H // 32) % (2 * S) == 0:
        S *= 2
    steps = H // 32 // S
    return S, steps, min(steps, 4)


def emu_router_mfma(x, w, bias, S, steps, nw, bf16_act=True):
    """The matrix-core router (batches of 16+ tokens): slice z holds steps of
    32 columns; wave v takes steps v, v + nw, ... in order, one matrix-core
    instruction per step (two with bf16 activations: the fp16 weight enters
    as an exact bf16 hi + lo pair); the wave partials are added in wave order,
    the slices in slice order (in the top-k kernel), then the bias."""
    slices = []
    for z in range(S):
        waves = []
        for v in range(nw):
            acc = P(0.0)
            for st in range(v, steps, nw):
                cols = range(32 * (z * steps + st), 32 * (z * steps + st) + 32)
                if bf16_act:
                    # fp16 weight = bf16 truncation + bf16 remainder (exact)
                    parts = []
                    for c in cols:
                        wf = np.float32(w[c])
                        hi = (np.array([wf], np.float32).view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)[0]
                        parts.append((hi, np.float32(wf - hi)))
                    halves = ([p[0] for p in parts], [p[1] for p in parts])
                else:
                    halves = ([w[c] for c in cols],)
                for ws in halves:
                    s = prod(x[cols[0]], ws[0])
                    for c, wc in zip(cols[1:], ws[1:]):
                        s = add(s, prod(x[c], wc))
                    acc = add(acc, s)
            waves.append(acc)
        tot = P(0.0)
        for wv in waves:
            tot = add(tot, wv)
        slices.append(tot)
    z = slices[0]
    for s in slices[1:]:
        z = add(z, s)
    if bias is not None:
        z = add(z, P(np.float32(bias)))
    return z


def exact_logit(x, w, bias):
    from fractions import Fraction
    s = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x, w)), Fraction(0))
    if bias is not None:
        s += Fraction(float(np.float32(bias)))
    return s


def check_row(x, w, bias, emu):
    from fractions import Fraction
    z = emu(x, w, bias)
    err = abs(Fraction(float(z.v)) - exact_logit(x, w, bias))
    wr = np.stack([np.asarray(w, np.float64), np.zeros(len(w))])
    b = None if bias is None else np.array([np.float64(np.float32(bias))])
    bound = mo.logit_error_bound(np.asarray(x, np.float64), wr, b, 0)
    assert z.d <= 64, f"summation depth {z.d} exceeds the bound's 64"
    assert float(err) <= bound, f"fp32 error {float(err):.3e} exceeds the bound {bound:.3e}"
    return float(err), bound, z.d


def bf16(v):
    return mo.bf16_bits_to_f64(mo.f64_to_bf16_bits_rne(np.asarray(v, np.float64)))


def f16(v):
    return np.asarray(v, np.float64).astype(np.float16).astype(np.float64)


def adversarial_same_sign(H):
    """Lane 0 of the per-row router: 1.0 first, then 31 products of 0.75 u,
    each of which the running sum near 1 (ulp 2u) rounds away."""
    x = np.zeros(H)
    w = np.zeros(H)
    cols = [512 * it + i for it in range((H + 511) // 512) for i in range(8)]
    x[cols[0]], w[cols[0]] = 1.0, 1.0
    for c in cols[1:]:
        x[c], w[c] = 3.0 * 2.0 ** -13, 2.0 ** -13      # product 3 * 2^-26 = 0.75 u
    return x, w


def test_bound_is_reached_within_a_factor_four_on_an_adversarial_row():
    x, w = adversarial_same_sign(2048)
    err, bound, depth = check_row(x, w, None, emu_router_vector)
    assert err == pytest.approx(31 * 0.75 * U, rel=1e-9)
    assert err >= bound / 4, f"bound {bound:.3e} is more than 4x the reachable error {err:.3e}"
    assert depth == 32 + 6


def test_heavy_cancellation_rows():
    rng = np.random.default_rng(21)
    for H in (256, 2048):
        for _ in range(3):
            big = bf16(rng.uniform(1.0, 2.0, H // 2))
            x = np.empty(H)
            x[0::2], x[1::2] = big, -big           # pairs cancel exactly in exact arithmetic
            x[1::2] = bf16(x[1::2] * (1 + 2.0 ** -7 * rng.integers(-1, 2, H // 2)))
            w = f16(rng.uniform(0.5, 1.0, H))
            bias = np.float32(rng.standard_normal())
            check_row(x, w, bias, emu_router_vector)
            S, steps, nw = router_slices(H, 512, 64)
            check_row(x, w, bias, lambda a, b, c: emu_router_mfma(a, b, c, S, steps, nw))


def test_same_sign_rows_both_orders():
    rng = np.random.default_rng(22)
    for H in (320, 2048):
        x = bf16(np.abs(rng.standard_normal(H)) + 0.5)
        w = f16(rng.uniform(0.01, 0.05, H))
        check_row(x, w, np.float32(3.5), emu_router_vector)
        S, steps, nw = router_slices(H, 512, 64)
        check_row(x, w, np.float32(3.5), lambda a, b, c: emu_router_mfma(a, b, c, S, steps, nw))
        check_row(x, w, None, lambda a, b, c: emu_router_mfma(a, b, c, S, steps, nw, bf16_act=False))


def test_workload_rows_and_depths():
    # rows of the 80B workload: x ~ N(0,1) bf16, router weights fp16 N(0, 1/sqrt(2048)), Zipf-sized bias
    rng = np.random.default_rng(23)
    H = 2048
    S, steps, nw = router_slices(H, 512, 64)
    assert (S, steps, nw) == (2, 32, 4)
    depths = set()
    for _ in range(4):
        x = bf16(rng.standard_normal(H))
        w = f16(rng.standard_normal(H) / math.sqrt(H))
        bias = np.float32(-1.3 * math.log(1 + rng.integers(0, 512)))
        depths.add(check_row(x, w, bias, emu_router_vector)[2])
        depths.add(check_row(x, w, bias, lambda a, b, c: emu_router_mfma(a, b, c, S, steps, nw))[2])
    # per-row: 32 sequential + 6 butterfly + bias; matrix cores: 31 inside an
    # instruction + 16 instructions + 4 waves + 1 slice + bias
    assert depths == {39, 53}


def test_a_bound_that_drops_the_depth_fails():
    # a plausible mistake (bound with one rounding per term instead of the
    # tree depth) is caught by the adversarial row
    x, w = adversarial_same_sign(2048)
    z = emu_router_vector(x, w, None)
    err = abs(float(z.v) - float(exact_logit(x, w, None)))
    wrong = 1.0 * U * float(np.abs(x * w).sum())
    assert err > wrong
