"""Shared helpers of the GPU parity tests: build device layers from the seeded
generator, run the fp64 oracle on the same inputs, compare."""
from __future__ import annotations

import math

import numpy as np

import synth
from oracle import moe_oracle as mo


def torch_mod():
    import torch
    return torch


def desc_for(wl, path=0, act=None, shared_inter=None):
    from int4_routed_expert_router_amd.api import Desc
    return Desc(wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter if shared_inter is None else shared_inter,
                wl.group, act or wl.act_dtype, path, wl.bits)


class DeviceLayer:
    """One layer's weights on the GPU plus what the oracle needs to regenerate them."""

    def __init__(self, wl, layer, use_gpu_fill=True, general_bias_seed=None, shared=True, router_scale=1.0,
                 bias_epoch=0, dup_rows=None):
        import torch
        from int4_routed_expert_router_amd import api
        self.wl, self.layer = wl, layer
        self.general_bias_seed = general_bias_seed
        h = wl.hidden
        self.stride = api.blob_bytes(h, wl.inter, wl.group, wl.bits)
        wr = synth.router_weights(wl, layer)
        if router_scale != 1.0:
            wr = synth.f32_to_f16_bits(wr.view(np.float16).astype(np.float32) * np.float32(router_scale))
        if dup_rows is not None:
            for dst, src in dup_rows:
                wr[dst] = wr[src]
        self.router_bits = wr
        self.bias = synth.router_bias(wl, layer, epoch=bias_epoch)
        self.router_w = torch.from_numpy(wr.view(np.int16).copy()).cuda()
        self.router_bias = None if self.bias is None else torch.from_numpy(self.bias.copy()).cuda()
        self.experts = torch.empty(wl.n_experts * self.stride, dtype=torch.uint8, device="cuda")
        if use_gpu_fill and general_bias_seed is None:
            api.synth_fill_experts(wl.weight_seed, layer, 0, wl.n_experts, h, wl.inter, wl.group, wl.scale_lo,
                                   wl.scale_hi, self.experts, self.stride, bits=wl.bits)
        else:
            host = np.zeros(wl.n_experts * self.stride, np.uint8)
            for e in range(wl.n_experts):
                host[e * self.stride:(e + 1) * self.stride] = api.pack_expert(self.raw(e), h, wl.inter, wl.group,
                                                                              wl.bits)
            self.experts.copy_(torch.from_numpy(host))
        self.has_shared = shared and wl.shared_inter > 0
        self.shared = None
        if self.has_shared:
            sb = api.blob_bytes(h, wl.shared_inter, wl.group, wl.bits)
            self.shared = torch.empty(sb, dtype=torch.uint8, device="cuda")
            if use_gpu_fill and general_bias_seed is None:
                api.synth_fill_experts(wl.weight_seed, layer, wl.n_experts, 1, h, wl.shared_inter, wl.group,
                                       wl.scale_lo, wl.scale_hi, self.shared, sb, bits=wl.bits)
            else:
                self.shared.copy_(torch.from_numpy(api.pack_expert(self.raw(0, shared=True), h, wl.shared_inter,
                                                                   wl.group, wl.bits)))
        self._cache = {}

    def raw(self, e, shared=False):
        r = synth.expert_raw(self.wl, self.layer, e, shared=shared)
        if self.general_bias_seed is not None:
            r = synth.random_affine_bias(r, self.general_bias_seed + 7919 * e + (104729 if shared else 0),
                                         bits=self.wl.bits)
        return r

    def api_layer(self):
        from int4_routed_expert_router_amd.api import Layer
        return Layer(self.router_w, self.router_bias, self.experts, self.stride, None, self.shared)

    def oracle_expert(self, e):
        if e not in self._cache:
            r = self.raw(e)
            self._cache[e] = mo.ExpertWeights.from_quant(r["gate"], r["up"], r["down"], self.wl.group, self.wl.bits)
        return self._cache[e]

    def oracle_shared(self):
        if not self.has_shared:
            return None
        if "s" not in self._cache:
            r = self.raw(0, shared=True)
            self._cache["s"] = mo.ExpertWeights.from_quant(r["gate"], r["up"], r["down"], self.wl.group,
                                                           self.wl.bits)
        return self._cache["s"]

    def router_f64(self):
        return mo.f16_bits_to_f64(self.router_bits)

    def bias_f64(self):
        return None if self.bias is None else self.bias.astype(np.float64)


def assert_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    tol = mo.tolerance(ref)
    err = np.abs(gpu - ref)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{what}: max |gpu - oracle| = {worst:.3e} > tol {tol:.3e}"
    return worst, tol


def check_routing(gpu_idx, gpu_w, gpu_logits, x64, wr64, bias64, k):
    """Returns the index sets the oracle should use per token and the number of
    near-tie tokens.

    (i) the GPU's top-k of its own fp32 logits equals the oracle's ordering of
        those same values, bit for bit, always;
    (ii) against the fp64 logits the sets agree unless the K-th/(K+1)-th gap is
        below the fp32 error bound of the two boundary logits; such tokens are
        counted, must differ only at the boundary, and are then compared
        against the oracle evaluated on the GPU's set.
    """
    n_t = gpu_idx.shape[0]
    z64, _ = mo.router_logits(x64, wr64, bias64)
    sets = []
    flagged = 0
    for t in range(n_t):
        own = mo.topk_order(gpu_logits[t, :-1].astype(np.float64), k)
        assert own.tolist() == gpu_idx[t].tolist(), f"token {t}: GPU top-k differs from its own logits' order"
        ref = mo.topk_order(z64[t], k)
        if ref.tolist() == gpu_idx[t].tolist():
            sets.append(ref)
            continue
        # allowed only for near ties: every position where the orders differ
        # must involve logits closer than the fp32 error bound
        bnd = {int(e): mo.logit_error_bound(x64[t], wr64, bias64, int(e)) for e in set(ref) | set(gpu_idx[t])}
        order = np.lexsort((np.arange(z64.shape[1]), -z64[t]))
        extra = int(order[k]) if k < len(order) else -1
        if extra >= 0:
            bnd[extra] = mo.logit_error_bound(x64[t], wr64, bias64, extra)
        for a, b in zip(ref.tolist(), gpu_idx[t].tolist()):
            if a != b:
                gap = abs(z64[t, a] - z64[t, b])
                eb = bnd.get(a, 0) + mo.logit_error_bound(x64[t], wr64, bias64, b)
                assert gap <= eb, f"token {t}: index {a} vs {b} differ with gap {gap:.3e} > bound {eb:.3e}"
        flagged += 1
        sets.append(np.asarray(gpu_idx[t]))
    return np.stack(sets), flagged


def bf16_to_f64(t):
    return mo.bf16_bits_to_f64(t.cpu().numpy().view(np.uint16))


def act_to_f64(t, act):
    return mo.act_bits_to_f64(t.cpu().numpy().view(np.uint16), act)


def rel(a, b):
    return float(np.abs(np.asarray(a) - np.asarray(b)).max() / max(1e-30, np.abs(np.asarray(b)).max()))


def isclose_rel(a, b, r):
    return math.isclose(a, b, rel_tol=r)
