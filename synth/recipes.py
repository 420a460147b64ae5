"""Seeded synthetic inputs for the routed MoE block.

This module only produces inputs; it holds none of the method's arithmetic
(no dequantisation, products, routing or combining).  Both the fp64 oracle
and the HIP path are fed from it.

Workloads (shapes from the pages' two model sizes: 8 of 256 experts for the
35B and 10 of 512 for the 80B, Show HN page, how-it-works list):

  tiny     H=256,  E=16,  K=2,  I=I_s=64,  G=32, T=4,  L=1,  fp16 activations
  dec35    H=2048, E=256, K=8,  I=I_s=512, G=64, T=1,  L=40, bf16
  dec80    H=2048, E=512, K=10, I=I_s=512, G=64, T=1,  L=48, bf16
  bat80    dec80 weights, T=64, Zipf exponent 1.3
  pool80   dec80 weights as pinned host blobs, 128 HBM slots per layer,
           T=1 for 256 steps, bias permutation redrawn every 32 steps,
           router weights x3 (logit noise sigma 3; measured hit rate 66%)
  dec80i8  dec80 shapes with int8 experts (the pages' other affine variant),
           scales U(1e-4, 1e-3) so that weights span the int4 range
  bat80i8  bat80 with the int8 experts of dec80i8

Expert weights (the bulk: 43.5 GB at the 80B shape) come from Philox4x32-10
so that any single expert can be regenerated alone, here or on the GPU:

  key     = (seed & 0xffffffff, layer)
  counter = (block, expert, tensor, 0), expert = E for the shared expert,
            tensor 0/1/2 = gate/up/down nibbles, 3/4/5 = gate/up/down scales
  nibbles : value j = r*cols + c of a [rows, cols] matrix is bits
            [4*(j%8), 4*(j%8)+4) of word (j%32)//8 of block j//32
  bytes   : (int8 experts) value j is bits [8*(j%4), 8*(j%4)+8) of word
            (j%16)//4 of block j//16
  scales  : value j = r*ngroups + g takes word j%4 of block j//4,
            u = (word >> 8) * 2**-24, s = fp16_rne(fl32(fl32(u*span) + lo))
            with fp32 constants lo and span = fl32(hi - lo); b = -8*s, or
            -128*s for int8 (exact either way)

Router weights, shared-gate vectors, router bias and tokens are small and are
drawn on the host with numpy's SeedSequence/PCG64 streams keyed by
(seed, layer, tag).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from .philox import philox4x32_10

T_GATE_Q, T_UP_Q, T_DOWN_Q, T_GATE_S, T_UP_S, T_DOWN_S = range(6)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    group: int
    tokens: int
    layers: int
    act_dtype: str            # "f16" | "bf16"
    weight_seed: int
    token_seed: int
    scale_lo: float
    scale_hi: float
    router_sigma: float       # std of router / shared-gate weights
    zipf_s: float             # 0 = no router bias
    slots_per_layer: int = 0  # pool workload only
    steps: int = 1
    drift_period: int = 0
    drift_seed: int = 0
    bits: int = 4             # expert weight width: 4 or 8

    @property
    def blob_bytes(self) -> int:
        h, i, g = self.hidden, self.inter, self.group
        return 3 * i * h * self.bits // 8 + 12 * i * h // g

    @property
    def shared_blob_bytes(self) -> int:
        h, i, g = self.hidden, self.shared_inter, self.group
        return 3 * i * h * self.bits // 8 + 12 * i * h // g


TINY = Workload("tiny", 256, 16, 2, 64, 64, 32, 4, 1, "f16", 0, 100, 0.002, 0.01, 0.02, 0.0)
DEC35 = Workload("dec35", 2048, 256, 8, 512, 512, 64, 1, 40, "bf16", 1, 101, 0.001, 0.01,
                 1.0 / math.sqrt(2048), 1.1)
DEC80 = Workload("dec80", 2048, 512, 10, 512, 512, 64, 1, 48, "bf16", 2, 102, 0.001, 0.01,
                 1.0 / math.sqrt(2048), 1.1)
BAT80 = dataclasses.replace(DEC80, name="bat80", tokens=64, token_seed=103, zipf_s=1.3)
POOL80 = dataclasses.replace(DEC80, name="pool80", token_seed=104, slots_per_layer=128, steps=256,
                             drift_period=32, drift_seed=105, router_sigma=3.0 / math.sqrt(2048))
DEC80I8 = dataclasses.replace(DEC80, name="dec80i8", bits=8, scale_lo=1e-4, scale_hi=1e-3)
BAT80I8 = dataclasses.replace(BAT80, name="bat80i8", bits=8, scale_lo=1e-4, scale_hi=1e-3)
WORKLOADS = {w.name: w for w in (TINY, DEC35, DEC80, BAT80, POOL80, DEC80I8, BAT80I8)}


@dataclasses.dataclass(frozen=True)
class GdnWorkload:
    """Gated DeltaNet decode step beside the MoE block (the pages give no sizes;
    these follow the public Qwen3-Next-80B configuration: 32 value heads and 16
    key heads of 128 dims, 36 of the 48 layers)."""
    name: str
    batch: int
    k_heads: int
    v_heads: int
    head_k_dim: int
    head_v_dim: int
    layers: int
    act_dtype: str
    seed: int


GDN80 = GdnWorkload("gdn80", 64, 16, 32, 128, 128, 36, "bf16", 201)
GDN_TINY = GdnWorkload("gdn_tiny", 3, 2, 4, 128, 32, 1, "f16", 202)


# ---------------------------------------------------------------------------
# rounding of generated fp32 draws to the stored 16-bit formats
# ---------------------------------------------------------------------------


def f32_to_f16_bits(v) -> np.ndarray:
    """Round-to-nearest-even fp32 -> fp16 (numpy's conversion is RNE)."""
    return np.asarray(v, dtype=np.float32).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(v) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 for finite values."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


# ---------------------------------------------------------------------------
# expert weights (Philox streams)
# ---------------------------------------------------------------------------


def _nibbles(seed: int, layer: int, expert: int, tensor: int, rows: int, cols: int) -> np.ndarray:
    n = rows * cols
    if n % 32:
        raise ValueError("rows*cols must be a multiple of 32")
    blocks = np.arange(n // 32, dtype=np.uint32)
    words = philox4x32_10(blocks, expert, tensor, 0, seed & 0xFFFFFFFF, layer)
    w = np.stack(words, axis=1)                                   # [blocks, 4]
    shifts = (4 * np.arange(8)).astype(np.uint32)
    vals = (w[:, :, None] >> shifts) & np.uint32(0xF)             # [blocks, 4, 8]
    return vals.reshape(rows, cols).astype(np.uint8)


def _bytes(seed: int, layer: int, expert: int, tensor: int, rows: int, cols: int) -> np.ndarray:
    n = rows * cols
    if n % 16:
        raise ValueError("rows*cols must be a multiple of 16")
    blocks = np.arange(n // 16, dtype=np.uint32)
    words = philox4x32_10(blocks, expert, tensor, 0, seed & 0xFFFFFFFF, layer)
    w = np.stack(words, axis=1)                                   # [blocks, 4]
    shifts = (8 * np.arange(4)).astype(np.uint32)
    vals = (w[:, :, None] >> shifts) & np.uint32(0xFF)            # [blocks, 4, 4]
    return vals.reshape(rows, cols).astype(np.uint8)


def _scales(seed: int, layer: int, expert: int, tensor: int, rows: int, ngroups: int,
            lo: float, hi: float, bits: int = 4):
    n = rows * ngroups
    nblocks = (n + 3) // 4
    blocks = np.arange(nblocks, dtype=np.uint32)
    words = np.stack(philox4x32_10(blocks, expert, tensor, 0, seed & 0xFFFFFFFF, layer), axis=1).reshape(-1)[:n]
    u = (words >> np.uint32(8)).astype(np.float32) * np.float32(2.0 ** -24)
    lo32 = np.float32(lo)
    span32 = np.float32(hi - lo)
    s32 = (u * span32).astype(np.float32) + lo32
    s16 = s32.astype(np.float32).astype(np.float16)
    b16 = (s16 * np.float16(-float(1 << (bits - 1)))).astype(np.float16)   # exact: power-of-two multiple
    return s16.view(np.uint16).reshape(rows, ngroups), b16.view(np.uint16).reshape(rows, ngroups)


def expert_raw(wl: Workload, layer: int, expert: int, shared: bool = False, seed: int | None = None):
    """Raw quantised tensors of one expert: dict(gate=(q,s,b), up=..., down=...).

    gate/up q: [I, H] uint8 in 0..2**bits - 1; down q: [H, I]; s, b: fp16 bit
    patterns [rows, cols // G].  ``expert`` is ignored for the shared expert
    (id E).
    """
    seed = wl.weight_seed if seed is None else seed
    h = wl.hidden
    i = wl.shared_inter if shared else wl.inter
    g = wl.group
    eid = wl.n_experts if shared else expert
    out = {}
    for name, tq, ts, rows, cols in (("gate", T_GATE_Q, T_GATE_S, i, h),
                                     ("up", T_UP_Q, T_UP_S, i, h),
                                     ("down", T_DOWN_Q, T_DOWN_S, h, i)):
        q = (_bytes if wl.bits == 8 else _nibbles)(seed, layer, eid, tq, rows, cols)
        s, b = _scales(seed, layer, eid, ts, rows, cols // g, wl.scale_lo, wl.scale_hi, wl.bits)
        out[name] = (q, s, b)
    return out


def random_affine_bias(raw, seed: int, bits: int = 4):
    """Replace b = -2**(bits-1)*s with general affine biases b = fp16(-s * U(0, 2**bits - 1)).

    Used by tests to exercise arbitrary per-group biases.
    """
    rng = np.random.default_rng([seed, 0xB1A5])
    top = float((1 << bits) - 1)
    out = {}
    for name, (q, s, _) in raw.items():
        sv = s.view(np.float16).astype(np.float32)
        b = (-sv * rng.uniform(0.0, top, size=s.shape).astype(np.float32)).astype(np.float16)
        out[name] = (q, s, b.view(np.uint16))
    return out


# ---------------------------------------------------------------------------
# router, bias, tokens (host numpy streams)
# ---------------------------------------------------------------------------

TAG_ROUTER, TAG_BIAS, TAG_TOKENS, TAG_DRIFT, TAG_GDN, TAG_GDN_STATE = 1, 2, 3, 4, 5, 6


def router_weights(wl: Workload, layer: int, seed: int | None = None) -> np.ndarray:
    """[E + 1, H] fp16 bit patterns; row E is the shared-gate vector."""
    seed = wl.weight_seed if seed is None else seed
    rng = np.random.default_rng([seed, layer, TAG_ROUTER])
    v = rng.standard_normal((wl.n_experts + 1, wl.hidden), dtype=np.float32) * np.float32(wl.router_sigma)
    return f32_to_f16_bits(v)


def zipf_bias(n_experts: int, s: float, perm: np.ndarray) -> np.ndarray:
    """beta_e = -s * ln(1 + perm[e]) as fp32 (softmax of beta alone is Zipf(s))."""
    rank = 1.0 + perm.astype(np.float64)
    return (-s * np.log(rank)).astype(np.float32)


def router_bias(wl: Workload, layer: int, epoch: int = 0, seed: int | None = None):
    """[E] fp32 Zipf bias for a layer (None when the workload has none).

    With drift, epoch k (steps k*period .. ) draws its own permutation.
    """
    if wl.zipf_s == 0.0:
        return None
    if epoch == 0:
        seed = wl.weight_seed if seed is None else seed
        rng = np.random.default_rng([seed, layer, TAG_BIAS])
    else:
        rng = np.random.default_rng([wl.drift_seed, layer, epoch, TAG_DRIFT])
    perm = rng.permutation(wl.n_experts)
    return zipf_bias(wl.n_experts, wl.zipf_s, perm)


def tokens(wl: Workload, n_tokens: int | None = None, seed: int | None = None, step: int = 0) -> np.ndarray:
    """[T, H] activation bit patterns (fp16 or bf16, RNE from fp32 N(0,1))."""
    n_tokens = wl.tokens if n_tokens is None else n_tokens
    seed = wl.token_seed if seed is None else seed
    rng = np.random.default_rng([seed, step, TAG_TOKENS])
    v = rng.standard_normal((n_tokens, wl.hidden), dtype=np.float32)
    return f32_to_f16_bits(v) if wl.act_dtype == "f16" else f32_to_bf16_bits(v)


# ---------------------------------------------------------------------------
# Gated DeltaNet step inputs (host numpy streams)
# ---------------------------------------------------------------------------


def gdn_inputs(wl: GdnWorkload, layer: int, step: int, batch: int | None = None):
    """One token's q, k [B, Hk, dk] and v [B, Hv, dv] as activation bit patterns
    (RNE from fp32 N(0,1)), the log-gate g [B, Hv] fp32 with exp(g) ~ U(0.85, 1)
    and beta [B, Hv] fp32 ~ U(0, 1)."""
    b = wl.batch if batch is None else batch
    rng = np.random.default_rng([wl.seed, layer, step, TAG_GDN])
    to_bits = f32_to_f16_bits if wl.act_dtype == "f16" else f32_to_bf16_bits
    q = to_bits(rng.standard_normal((b, wl.k_heads, wl.head_k_dim), dtype=np.float32))
    k = to_bits(rng.standard_normal((b, wl.k_heads, wl.head_k_dim), dtype=np.float32))
    v = to_bits(rng.standard_normal((b, wl.v_heads, wl.head_v_dim), dtype=np.float32))
    g = np.log(rng.uniform(0.85, 1.0, (b, wl.v_heads))).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (b, wl.v_heads)).astype(np.float32)
    return q, k, v, g, beta


def gdn_state(wl: GdnWorkload, layer: int, batch: int | None = None) -> np.ndarray:
    """An initial recurrent state [B, Hv, dv, dk] fp32 ~ N(0, 0.05^2)."""
    b = wl.batch if batch is None else batch
    rng = np.random.default_rng([wl.seed, layer, TAG_GDN_STATE])
    shape = (b, wl.v_heads, wl.head_v_dim, wl.head_k_dim)
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(0.05)).astype(np.float32)
