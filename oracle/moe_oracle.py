"""fp64 reference of the routed MoE block (TEST INFRASTRUCTURE ONLY).

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
use this module; see the package docstring.  Parity status: pinned by
closed forms, brute force and invariants in tests/test_oracle_math.py;
absolute values at the 35B/80B shapes are "parity unpinned" beyond those.

The block (Qwen3-Next-style sparse MoE with a shared expert, the model family
of the Show HN page, intro and how-it-works list; the AIbase news page,
working-principle paragraph):

  z_e   = sum_h x_h * Wr[e,h] + beta_e           (router logits, e < E)
  z_s   = sum_h x_h * Wr[E,h]                     (shared-gate logit)
  S     = the K experts with the largest z, ordered by (z desc, index asc)
  w_k   = exp(z_{S_k} - z_{S_0}) / sum_j exp(z_{S_j} - z_{S_0})
          (softmax over all E followed by renormalisation over S reduces to
           exactly this, because the normalisers cancel)
  gamma = 1 / (1 + exp(-z_s))
  FFN(x; e) = Wd_e ( silu(Wg_e x) * (Wu_e x) ),  silu(a) = a / (1 + exp(-a))
  y     = sum_k w_k FFN(x; S_k) + gamma * FFN(x; shared)

Affine int4 weights (the MLX affine group quantisation named in the Show HN
page's what-was-built list): W[r, c] = s[r, c // G] * q[r, c] + b[r, c // G]
with q in 0..15 and fp16 s, b, groups of G columns along the input dimension.
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# exact decoding of the stored number formats
# ---------------------------------------------------------------------------


def f16_bits_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (upper half of a binary32) -> float64 (exact)."""
    wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(np.float64)


def act_bits_to_f64(bits, act_dtype: str) -> np.ndarray:
    if act_dtype == "f16":
        return f16_bits_to_f64(bits)
    if act_dtype == "bf16":
        return bf16_bits_to_f64(bits)
    raise ValueError(f"unknown activation dtype {act_dtype!r}")


def f64_to_bf16_bits_rne(v) -> np.ndarray:
    """Round float64 values to bfloat16 (round to nearest, ties to even).

    Written from the definition: a bfloat16 normal number carries 8
    significant bits, so v = m * 2**e with 0.5 <= |m| < 1 rounds to
    rint(m * 2**8) * 2**(e - 8) (numpy's rint is ties-to-even).  The result
    is exactly representable in binary32, whose upper 16 bits are the
    bfloat16 pattern.  Only finite values inside the bfloat16 normal range
    (or zero) are accepted.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite value")
    m, e = np.frexp(v)
    r = np.rint(m * 256.0) * np.exp2(e.astype(np.float64) - 8.0)
    nz = r != 0
    if np.any(np.abs(r[nz]) < 2.0 ** -126) or np.any(np.abs(r) >= 2.0 ** 128):
        raise ValueError("value outside the bfloat16 normal range")
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# affine int4 group dequantisation
# ---------------------------------------------------------------------------


def dequant(q, s_bits, b_bits, group: int, bits: int = 4) -> np.ndarray:
    """W[r, c] = s[r, c // G] * q[r, c] + b[r, c // G] in float64.

    q: [rows, cols] integers 0..2**bits - 1 (bits 4 or 8: the pages' affine
    int4 and int8 group quantisation); s_bits, b_bits: [rows, cols // G] fp16
    bit patterns.  Groups are G contiguous columns along the input dimension.
    """
    q = np.asarray(q)
    rows, cols = q.shape
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    if cols % group:
        raise ValueError("cols must be a multiple of the group size")
    if q.min(initial=0) < 0 or q.max(initial=0) > (1 << bits) - 1:
        raise ValueError(f"q must lie in 0..{(1 << bits) - 1}")
    s = f16_bits_to_f64(s_bits)
    b = f16_bits_to_f64(b_bits)
    if s.shape != (rows, cols // group) or b.shape != s.shape:
        raise ValueError("scale/bias shape mismatch")
    col_group = np.arange(cols) // group
    return s[:, col_group] * q.astype(np.float64) + b[:, col_group]


# ---------------------------------------------------------------------------
# router, top-k, weights, shared gate
# ---------------------------------------------------------------------------


def router_logits(x, router_w, bias=None):
    """Router GEMV with the shared-gate row fused in.

    x: [T, H] float64; router_w: [E + 1, H] float64 (row E is the shared-gate
    vector); bias: [E] float64 or None.  Returns (z [T, E], z_s [T]).
    """
    x = np.asarray(x, dtype=np.float64)
    wr = np.asarray(router_w, dtype=np.float64)
    n_e = wr.shape[0] - 1
    z = x @ wr[:n_e].T
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float64)[None, :]
    z_s = x @ wr[n_e]
    return z, z_s


def topk_order(z_row, k: int) -> np.ndarray:
    """Indices of the k largest values, ordered by (value desc, index asc).

    Equal values select the lower expert index first.
    """
    z_row = np.asarray(z_row, dtype=np.float64)
    if z_row.ndim != 1:
        raise ValueError("one row of logits expected")
    if not 1 <= k <= z_row.shape[0]:
        raise ValueError("k out of range")
    if np.any(np.isnan(z_row)):
        raise ValueError("NaN logits are not supported")
    idx = np.arange(z_row.shape[0])
    # lexsort orders by the last key first: primary -z ascending, then index.
    order = np.lexsort((idx, -z_row))
    return order[:k].astype(np.int64)


def renormalised_weights(z_selected) -> np.ndarray:
    """Softmax restricted to the selected logits (in rank order)."""
    z_sel = np.asarray(z_selected, dtype=np.float64)
    ex = np.exp(z_sel - z_sel.max())
    return ex / ex.sum()


def sigmoid(v):
    v = np.asarray(v, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-v))


def route(x, router_w, bias, k: int):
    """Router + top-k + renormalised weights + shared gate for T tokens.

    Returns (idx [T, K] int64, w [T, K], gamma [T], z [T, E], z_s [T]).
    """
    z, z_s = router_logits(x, router_w, bias)
    n_t = z.shape[0]
    idx = np.zeros((n_t, k), dtype=np.int64)
    w = np.zeros((n_t, k), dtype=np.float64)
    for t in range(n_t):
        idx[t] = topk_order(z[t], k)
        w[t] = renormalised_weights(z[t, idx[t]])
    return idx, w, sigmoid(z_s), z, z_s


def boundary_gap(z_row, k: int):
    """Gap between the K-th and (K+1)-th logit in oracle order (inf if K=E)."""
    order = np.lexsort((np.arange(len(z_row)), -np.asarray(z_row, np.float64)))
    if k >= len(z_row):
        return math.inf, int(order[k - 1]), -1
    return float(z_row[order[k - 1]] - z_row[order[k]]), int(order[k - 1]), int(order[k])


def logit_error_bound(x_row, router_w, bias, e: int) -> float:
    """Bound on |fp32 logit - exact logit| for a lane-blocked fp32 GEMV.

    Products of a 16-bit float activation with an fp16 weight are exact in
    binary32; a summation of depth d (the longest chain of fp32 additions
    any term passes through) adds at most d*u*sum|terms| (u = 2**-24).
    Depth 64 covers sequential runs of up to 32 terms followed by up to 31
    further additions (partial sums and the bias), which bounds every
    lane- or wave-blocked order of H <= 2048 terms used by the kernels.
    """
    terms = np.abs(np.asarray(x_row, np.float64) * np.asarray(router_w, np.float64)[e])
    extra = 0.0 if bias is None else abs(float(bias[e]))
    return 64.0 * 2.0 ** -24 * (float(terms.sum()) + extra)


# ---------------------------------------------------------------------------
# expert FFN and the layer
# ---------------------------------------------------------------------------


def silu(a):
    a = np.asarray(a, dtype=np.float64)
    return a / (1.0 + np.exp(-a))


def expert_ffn(x, wg, wu, wd, return_intermediates=False):
    """SwiGLU expert: y = Wd (silu(Wg x) * (Wu x)) for x [T, H] (float64).

    wg, wu: [I, H]; wd: [H, I] (dequantised float64 matrices).
    """
    x = np.asarray(x, dtype=np.float64)
    a = x @ np.asarray(wg, np.float64).T
    u = x @ np.asarray(wu, np.float64).T
    h = silu(a) * u
    y = h @ np.asarray(wd, np.float64).T
    if return_intermediates:
        return y, a, u, h
    return y


class ExpertWeights:
    """Dequantised float64 matrices of one expert (gate, up: [I, H]; down: [H, I])."""

    def __init__(self, wg, wu, wd):
        self.wg = np.asarray(wg, np.float64)
        self.wu = np.asarray(wu, np.float64)
        self.wd = np.asarray(wd, np.float64)

    @classmethod
    def from_quant(cls, gate, up, down, group: int, bits: int = 4):
        """Each of gate/up/down is a (q, s_bits, b_bits) triple."""
        return cls(dequant(*gate, group, bits), dequant(*up, group, bits), dequant(*down, group, bits))


def combine(w_row, expert_outputs, gamma, shared_output):
    """y = sum_k w_k * y_k (k in rank order) + gamma * y_shared."""
    y = np.zeros_like(np.asarray(shared_output, np.float64))
    for wk, yk in zip(w_row, expert_outputs):
        y = y + wk * np.asarray(yk, np.float64)
    return y + gamma * np.asarray(shared_output, np.float64)


def layer_forward(x, router_w, bias, experts, shared, k: int, forced_idx=None):
    """The MoE block for T tokens.

    x: [T, H] float64; router_w: [E+1, H] float64; bias: [E] or None;
    experts: callable e -> ExpertWeights (only the selected ones are touched);
    shared: ExpertWeights or None (no shared expert: gamma term dropped).
    forced_idx: optional [T, K] index sets to use instead of the oracle's own
    top-k (used where an fp32 near-tie legitimately picks a different set;
    the weights are then the renormalised softmax over that set).

    Returns dict(y [T, H], idx, w, gamma, z, z_s).
    """
    x = np.asarray(x, dtype=np.float64)
    idx, w, gamma, z, z_s = route(x, router_w, bias, k)
    if forced_idx is not None:
        idx = np.asarray(forced_idx, dtype=np.int64).copy()
        for t in range(x.shape[0]):
            w[t] = renormalised_weights(z[t, idx[t]])
    cache = {}
    y = np.zeros_like(x)
    for t in range(x.shape[0]):
        outs = []
        for e in idx[t]:
            e = int(e)
            if e not in cache:
                cache[e] = experts(e)
            ew = cache[e]
            outs.append(expert_ffn(x[t:t + 1], ew.wg, ew.wu, ew.wd)[0])
        if shared is not None:
            ys = expert_ffn(x[t:t + 1], shared.wg, shared.wu, shared.wd)[0]
            g = gamma[t]
        else:
            ys = np.zeros(x.shape[1])
            g = 0.0
        y[t] = combine(w[t], outs, g, ys)
    return dict(y=y, idx=idx, w=w, gamma=gamma, z=z, z_s=z_s)


def layer_forward_dense(x, router_w, bias, all_experts, shared, k: int):
    """Same block computed densely: every expert runs, and the combine uses a
    length-E weight vector that is zero outside the selected set.  Used only
    to cross-check the sparse gather/index logic of ``layer_forward``.
    """
    x = np.asarray(x, dtype=np.float64)
    idx, w, gamma, z, _ = route(x, router_w, bias, k)
    n_t, n_e = z.shape
    dense_w = np.zeros((n_t, n_e))
    for t in range(n_t):
        dense_w[t, idx[t]] = w[t]
    outs = np.stack([expert_ffn(x, ew.wg, ew.wu, ew.wd) for ew in all_experts], axis=1)  # [T,E,H]
    y = np.einsum("te,teh->th", dense_w, outs)
    if shared is not None:
        y = y + gamma[:, None] * expert_ffn(x, shared.wg, shared.wu, shared.wd)
    return y


# ---------------------------------------------------------------------------
# stack chaining (pre-norm residual stand-in between MoE layers)
# ---------------------------------------------------------------------------

RMS_EPS = 1e-6


def stack_epilogue(r, y):
    """r' = r + y; next-layer input x' = bf16_rne(r' / sqrt(mean(r'^2) + eps)).

    r, y: [T, H].  Returns (r' float64, x' bf16 bit patterns uint16).
    """
    r_new = np.asarray(r, np.float64) + np.asarray(y, np.float64)
    rms = np.sqrt(np.mean(r_new * r_new, axis=1, keepdims=True) + RMS_EPS)
    return r_new, f64_to_bf16_bits_rne(r_new / rms)


def tolerance(ref) -> float:
    """Per-element bound |gpu - oracle| <= 1e-3 * max|oracle| + 1e-5."""
    ref = np.asarray(ref, np.float64)
    return 1e-3 * (float(np.abs(ref).max()) if ref.size else 0.0) + 1e-5
