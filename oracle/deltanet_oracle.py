"""Gated DeltaNet single-token recurrence in float64 (TEST INFRASTRUCTURE ONLY).

The pages state that three quarters of the layers of these hybrid models use
Gated DeltaNet linear attention with a fixed-size recurrent state (Show HN
page, how-it-works list; aibase article, working principle), and give nothing
more.  The recurrence here is the published gated delta rule (Yang, Kautz and
Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with Delta Rule", ICLR
2025), per value head, with S a [d_v, d_k] matrix:

    k^ = k / sqrt(|k|^2 + eps),   q^ = q_scale * q / sqrt(|q|^2 + eps)
    alpha = exp(g)  (g <= 0, the gate),   beta in [0, 1]
    S_t = S_{t-1} (alpha (I - beta k^ k^T)) + beta v k^T
        = alpha S_{t-1} + beta (v - alpha S_{t-1} k^) k^T
    o_t = S_t q^

Readings (the pages fix none of them): eps = 1e-6; value head h reads key
head h // (H_v / H_k) (consecutive value heads share a key head); the state
is kept in float32 by the kernel and float64 here.

Parity status: pinned in tests/test_oracle_deltanet.py by closed forms
(beta = 0, zero state, the delta rule's exact write at k^), the whole-sequence
matrix-product form of several steps, the head grouping and the invariance
under rescaling q and k.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def l2_normalise(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float64)
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + EPS)


def gdn_step(state, q, k, v, g, beta, q_scale: float):
    """One token for every sequence and value head.

    state [B, Hv, dv, dk]; q, k [B, Hk, dk]; v [B, Hv, dv]; g, beta [B, Hv].
    Returns (new_state, o [B, Hv, dv]), both float64; the inputs are not changed.
    """
    S = np.asarray(state, np.float64)
    B, Hv, dv, dk = S.shape
    Hk = q.shape[1]
    if Hv % Hk:
        raise ValueError("value heads must be a multiple of key heads")
    group = Hv // Hk
    kn = np.repeat(l2_normalise(k), group, axis=1)                  # [B, Hv, dk]
    qn = np.repeat(l2_normalise(q), group, axis=1) * q_scale        # [B, Hv, dk]
    alpha = np.exp(np.asarray(g, np.float64))[..., None]            # [B, Hv, 1]
    b = np.asarray(beta, np.float64)[..., None]
    sk = np.einsum("bhij,bhj->bhi", S, kn)                          # S k^
    delta = b * (np.asarray(v, np.float64) - alpha * sk)            # beta (v - alpha S k^)
    new = alpha[..., None] * S + delta[..., :, None] * kn[..., None, :]
    o = np.einsum("bhij,bhj->bhi", new, qn)
    return new, o
