"""Python binding of the C ABI (argument marshalling only).

Every step of the MoE path runs in the HIP library; PyTorch only provides
device memory (tensors) and streams.  Functions take torch tensors that
already live on the GPU and return nothing: outputs are written in place,
asynchronously on the current torch stream unless a stream is given.
"""
from __future__ import annotations

import ctypes as C
import dataclasses

import numpy as np
import torch

from ._lib import (GdnDesc, MOE_BF16, MOE_F16, MOE_PATH_AUTO, MOE_POOL_DMA_COPY, MOE_POOL_HOST_ONLY, LayerDesc,  # noqa: F401
                   LayerWeights, SlotPoolConfig, SlotPoolStats, check, lib)

__all__ = ["Desc", "Layer", "blob_bytes", "pack_expert", "workspace_bytes", "workspace", "route", "permute",
           "expert_ffn", "layer_forward", "stack_epilogue", "stack_forward", "StackGraph", "synth_fill_experts",
           "synth_philox", "SlotPool", "pool_decode_step", "gdn_step"]


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


@dataclasses.dataclass(frozen=True)
class Desc:
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    group_size: int
    act_dtype: str = "bf16"          # "f16" | "bf16"
    path: int = MOE_PATH_AUTO
    weight_bits: int = 4             # 4 | 8

    def c(self) -> LayerDesc:
        return LayerDesc(self.hidden, self.n_experts, self.top_k, self.inter, self.shared_inter, self.group_size,
                         {"bf16": MOE_BF16, "f16": MOE_F16}.get(self.act_dtype, 0), self.path, self.weight_bits)

    @property
    def blob_bytes(self) -> int:
        return blob_bytes(self.hidden, self.inter, self.group_size, self.weight_bits)

    @property
    def shared_blob_bytes(self) -> int:
        return blob_bytes(self.hidden, self.shared_inter, self.group_size, self.weight_bits) if self.shared_inter else 0


class Layer:
    """Device weights of one layer (keeps the tensors alive).

    router_w: [E+1, H] int16/uint16 fp16 bits; router_bias: [E] fp32 or None;
    experts: uint8 tensor holding the blobs (or an int device address);
    expert_stride: bytes; expert_offset: [E] int64 (uint64 semantics) or None;
    shared: uint8 blob tensor or None.
    """

    def __init__(self, router_w, router_bias, experts, expert_stride, expert_offset=None, shared=None):
        self.router_w, self.router_bias, self.experts = router_w, router_bias, experts
        self.expert_stride, self.expert_offset, self.shared = int(expert_stride), expert_offset, shared

    def c(self) -> LayerWeights:
        return LayerWeights(_ptr(self.router_w), _ptr(self.router_bias), _ptr(self.experts), self.expert_stride,
                            _ptr(self.expert_offset), _ptr(self.shared))


def blob_bytes(hidden: int, inter: int, group: int, bits: int = 4) -> int:
    return int(lib().moe_blob_bytes_q(hidden, inter, group, bits))


def pack_expert(raw, hidden: int, inter: int, group: int, bits: int = 4) -> np.ndarray:
    """Host packer: raw dict(gate=(q,s,b), up=..., down=...) -> blob bytes (np.uint8)."""
    out = np.zeros(blob_bytes(hidden, inter, group, bits), np.uint8)
    arrs = []
    for name in ("gate", "up", "down"):
        q, s, b = raw[name]
        arrs += [np.ascontiguousarray(q, np.uint8), np.ascontiguousarray(s, np.uint16),
                 np.ascontiguousarray(b, np.uint16)]
    check(lib().moe_pack_expert_q(hidden, inter, group, bits, *[a.ctypes.data for a in arrs], out.ctypes.data))
    return out


def workspace_bytes(desc: Desc, n_tokens: int) -> int:
    n = C.c_size_t(0)
    d = desc.c()
    check(lib().moe_workspace_bytes(C.byref(d), n_tokens, C.byref(n)))
    return int(n.value)


def workspace(desc: Desc, n_tokens: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(workspace_bytes(desc, n_tokens), 256), dtype=torch.uint8, device=device)


def route(desc, layer, x, topk_idx, topk_w, shared_gate=None, logits=None, ws=None, stream=None):
    d, w = desc.c(), layer.c()
    T = x.shape[0]
    ws = workspace(desc, T, x.device) if ws is None else ws
    check(lib().moe_route(C.byref(d), C.byref(w), _ptr(x), T, _ptr(topk_idx), _ptr(topk_w), _ptr(shared_gate),
                          _ptr(logits), _ptr(ws), ws.numel(), _stream(stream)))


def permute(desc, topk_idx, expert_off, perm, inv=None, ws=None, stream=None):
    d = desc.c()
    T = topk_idx.shape[0]
    ws = workspace(desc, T, topk_idx.device) if ws is None else ws
    check(lib().moe_permute(C.byref(d), _ptr(topk_idx), T, _ptr(expert_off), _ptr(perm), _ptr(inv), _ptr(ws),
                            ws.numel(), _stream(stream)))


def expert_ffn(desc, layer, x, topk_idx, topk_w, shared_gate, y, ws=None, stream=None):
    d, w = desc.c(), layer.c()
    T = x.shape[0]
    ws = workspace(desc, T, x.device) if ws is None else ws
    check(lib().moe_expert_ffn(C.byref(d), C.byref(w), _ptr(x), T, _ptr(topk_idx), _ptr(topk_w), _ptr(shared_gate),
                               _ptr(y), _ptr(ws), ws.numel(), _stream(stream)))


def layer_forward(desc, layer, x, y, topk_idx=None, topk_w=None, shared_gate=None, ws=None, stream=None):
    d, w = desc.c(), layer.c()
    T = x.shape[0]
    ws = workspace(desc, T, x.device) if ws is None else ws
    check(lib().moe_layer_forward(C.byref(d), C.byref(w), _ptr(x), T, _ptr(y), _ptr(topk_idx), _ptr(topk_w),
                                  _ptr(shared_gate), _ptr(ws), ws.numel(), _stream(stream)))


def stack_epilogue(desc, y, r, x_next, stream=None):
    d = desc.c()
    check(lib().moe_stack_epilogue(C.byref(d), y.shape[0], _ptr(y), _ptr(r), _ptr(x_next), _stream(stream)))


def _layer_array(layers):
    arr = (LayerWeights * len(layers))(*[l.c() for l in layers])
    return arr


def stack_forward(desc, layers, x0, r, x_buf, ws, x_all=None, y_all=None, idx_all=None, w_all=None,
                  gamma_all=None, stream=None):
    d = desc.c()
    arr = _layer_array(layers)
    check(lib().moe_stack_forward(C.byref(d), arr, len(layers), _ptr(x0), x0.shape[0], _ptr(r), _ptr(x_buf),
                                  _ptr(x_all), _ptr(y_all), _ptr(idx_all), _ptr(w_all), _ptr(gamma_all), _ptr(ws),
                                  ws.numel(), _stream(stream)))


class StackGraph:
    """moe_stack_forward captured once into a HIP graph; launch() replays it."""

    def __init__(self, desc, layers, x0, r, x_buf, ws, capture_stream, x_all=None, y_all=None, idx_all=None,
                 w_all=None, gamma_all=None):
        d = desc.c()
        arr = _layer_array(layers)
        h = C.c_void_p()
        self._keep = (layers, x0, r, x_buf, ws, x_all, y_all, idx_all, w_all, gamma_all)
        check(lib().moe_stack_graph_create(C.byref(d), arr, len(layers), _ptr(x0), x0.shape[0], _ptr(r), _ptr(x_buf),
                                           _ptr(x_all), _ptr(y_all), _ptr(idx_all), _ptr(w_all), _ptr(gamma_all),
                                           _ptr(ws), ws.numel(), _stream(capture_stream), C.byref(h)))
        self._h = h

    def launch(self, stream=None):
        check(lib().moe_graph_launch(self._h, _stream(stream)))

    def close(self):
        if self._h:
            lib().moe_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def pool_decode_step(desc, layers, pool, step, x0, r, x_buf, idx_host, ws, pregate=0, idx_log=None,
                     stream=None):
    """One batch-1 token through len(layers) layers streamed through `pool`
    (moe_pool_decode_step): x0 [1, H] or [H] device, r [H] fp32 device,
    x_buf [2, H] device, idx_host pinned int32 [2, K], pregate = predictions
    prefetched per layer (0 = none), idx_log optional host int32 numpy array
    [L, 2, K]."""
    d = desc.c()
    arr = _layer_array(layers)
    log = None if idx_log is None else idx_log.ctypes.data
    check(lib().moe_pool_decode_step(C.byref(d), arr, len(layers), pool._h, step, _ptr(x0), _ptr(r), _ptr(x_buf),
                                     _ptr(idx_host), log, int(pregate), _ptr(ws), ws.numel(),
                                     _stream(stream)))


def gdn_step(q, k, v, g, beta, state, o, q_scale, act_dtype="bf16", stream=None):
    """One Gated DeltaNet token (moe_gdn_step): q, k [B, Hk, 128] and v [B, Hv, dv]
    16-bit tensors, g, beta [B, Hv] fp32, state [B, Hv, dv, 128] fp32 (in place),
    o [B, Hv, dv] fp32."""
    B, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    d = GdnDesc(B, Hk, Hv, dk, dv, {"bf16": MOE_BF16, "f16": MOE_F16}.get(act_dtype, 0))
    check(lib().moe_gdn_step(C.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(q_scale), _ptr(state),
                             _ptr(o), _stream(stream)))


def synth_fill_experts(seed, layer, expert_first, n_experts, hidden, inter, group, scale_lo, scale_hi, dst, stride,
                       stream=None, bits: int = 4):
    """Fill blobs on the GPU with the seeded synthetic weights (see include/moe_synth.h)."""
    span = float(np.float32(scale_hi - scale_lo))
    check(lib().moe_synth_fill_experts(seed, layer, expert_first, n_experts, hidden, inter, group, bits,
                                       float(np.float32(scale_lo)), span, _ptr(dst), stride, _stream(stream)))


def synth_philox(ctr, key, out, stream=None):
    check(lib().moe_synth_philox(_ptr(ctr), _ptr(key), _ptr(out), ctr.shape[0], _stream(stream)))


class SlotPool:
    """Bounded HBM slot pool (include/moe_slotpool.h)."""

    def __init__(self, n_layers, n_experts, slots, aging_period, blob_stride=0, blob_bytes_=0, host_blobs=None,
                 device_slab=None, device_offsets=None, copy_stream=None, host_only=False, dma_copy=False):
        cfg = SlotPoolConfig(n_layers, n_experts, slots, aging_period, blob_stride, blob_bytes_, _ptr(host_blobs),
                             _ptr(device_slab), _ptr(device_offsets),
                             None if copy_stream is None else _stream(copy_stream),
                             (MOE_POOL_HOST_ONLY if host_only else 0) | (MOE_POOL_DMA_COPY if dma_copy else 0))
        h = C.c_void_p()
        check(lib().slotpool_create(C.byref(cfg), C.byref(h)))
        self._h = h
        self._keep = (host_blobs, device_slab, device_offsets, copy_stream)
        self.n_layers, self.n_experts, self.slots = n_layers, n_experts, slots

    def acquire(self, layer, experts, step, compute_stream=None):
        ex = np.ascontiguousarray(experts, dtype=np.int32)
        n = ex.size
        slot = np.zeros(n, np.int32)
        victim = np.zeros(n, np.int32)
        hit = np.zeros(n, np.uint8)
        cs = None if compute_stream is False else _stream(compute_stream)
        check(lib().slotpool_acquire(self._h, layer, ex.ctypes.data, n, step, cs, slot.ctypes.data,
                                     victim.ctypes.data, hit.ctypes.data))
        return [(int(e), bool(h), int(s), int(v)) for e, h, s, v in zip(ex, hit, slot, victim)]

    def prefetch(self, layer, experts, step, compute_stream=None):
        """Returns [(expert, slot, victim)] for the experts the call loaded."""
        ex = np.ascontiguousarray(experts, dtype=np.int32)
        n = ex.size
        n_loaded = C.c_int32(0)
        loaded, slot, victim = (np.zeros(max(n, 1), np.int32) for _ in range(3))
        cs = None if compute_stream is False else _stream(compute_stream)
        check(lib().slotpool_prefetch(self._h, layer, ex.ctypes.data, n, step, cs, C.byref(n_loaded),
                                      loaded.ctypes.data, slot.ctypes.data, victim.ctypes.data))
        k = n_loaded.value
        return [(int(e), int(s), int(v)) for e, s, v in zip(loaded[:k], slot[:k], victim[:k])]

    def release(self, layer, compute_stream=None):
        cs = None if compute_stream is False else _stream(compute_stream)
        check(lib().slotpool_release(self._h, layer, cs))

    def evict(self, layer, expert):
        check(lib().slotpool_evict(self._h, layer, expert))

    def stats(self):
        s = SlotPoolStats()
        check(lib().slotpool_stats(self._h, C.byref(s)))
        return dict(hits=s.hits, misses=s.misses, evictions=s.evictions, bytes_h2d=s.bytes_h2d,
                    prefetches=s.prefetches)

    def close(self):
        if self._h:
            lib().slotpool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
