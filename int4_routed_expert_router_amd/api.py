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

__all__ = ["Desc", "Layer", "blob_bytes", "pack_expert", "workspace_bytes", "workspace", "workspace_status",
           "route", "permute",
           "expert_ffn", "layer_forward", "layer_forward_static", "stack_epilogue", "stack_forward", "StackGraph", "synth_fill_experts",
           "synth_philox", "SlotPool", "pool_decode_step", "DevPool", "pool_decode_step_dev", "PoolGraph", "gdn_step"]


_ACT_DTYPES = (torch.int16, torch.float16, torch.bfloat16)


def _ptr(t, name="tensor", dtypes=None, numel=None, host=False):
    """Address of a tensor for the C ABI, after checking that it is where the
    call reads it (a CUDA tensor, or with host=True a CPU tensor),
    contiguous, of an accepted dtype and, when given, of numel elements.
    None stays NULL; a plain int is taken as an address the caller vouches
    for."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if host:
        if t.device.type != "cpu":
            raise ValueError(f"{name} must be a host (CPU) tensor, got {t.device}")
    elif t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _scratch(desc, T, device, stream):
    """A temporary workspace for one call.  It is allocated on the current
    stream; when the call runs on another torch stream the tensor is recorded
    on that stream too, so the caching allocator does not hand its memory out
    again before the call's kernels have finished with it."""
    if stream is not None and not isinstance(stream, torch.cuda.Stream):
        raise ValueError("pass ws explicitly when stream is a raw stream handle")
    ws = workspace(desc, T, device)
    if stream is not None and stream != torch.cuda.current_stream(ws.device):
        ws.record_stream(stream)
    return ws


def _tokens(x, desc, name="x"):
    if not isinstance(x, torch.Tensor) or x.dim() < 1:
        raise ValueError(f"{name} must be a [T, H] tensor")
    T = x.shape[0]
    _ptr(x, name, _ACT_DTYPES, T * desc.hidden)
    return T


def _ws(ws):
    return _ptr(ws, "ws", (torch.uint8,))


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
        return LayerWeights(_ptr(self.router_w, "router_w", (torch.int16, torch.float16)),
                            _ptr(self.router_bias, "router_bias", (torch.float32,)),
                            _ptr(self.experts, "experts", (torch.uint8,)), self.expert_stride,
                            _ptr(self.expert_offset, "expert_offset", (torch.int64,)),
                            _ptr(self.shared, "shared", (torch.uint8,)))


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


def workspace_status(desc: Desc, n_tokens: int, ws: torch.Tensor) -> int:
    """The status word (MOE_FLAG_* bits) the last call on ws left in it; the
    caller synchronises the call's stream first."""
    off = C.c_size_t(0)
    d = desc.c()
    check(lib().moe_workspace_status(C.byref(d), n_tokens, C.byref(off)))
    o = int(off.value)
    return int(ws[o:o + 4].view(torch.int32).item()) & 0xFFFFFFFF


_I32, _F32 = (torch.int32,), (torch.float32,)


def route(desc, layer, x, topk_idx, topk_w, shared_gate=None, logits=None, ws=None, stream=None):
    T = _tokens(x, desc)
    K, E = desc.top_k, desc.n_experts
    args = (_ptr(x), T, _ptr(topk_idx, "topk_idx", _I32, T * K), _ptr(topk_w, "topk_w", _F32, T * K),
            _ptr(shared_gate, "shared_gate", _F32, T), _ptr(logits, "logits", _F32, T * (E + 1)))
    d, w = desc.c(), layer.c()
    ws = _scratch(desc, T, x.device, stream) if ws is None else ws
    check(lib().moe_route(C.byref(d), C.byref(w), *args, _ws(ws), ws.numel(), _stream(stream)))


def permute(desc, topk_idx, expert_off, perm, inv=None, ws=None, stream=None):
    T = topk_idx.shape[0]
    K, E = desc.top_k, desc.n_experts
    args = (_ptr(topk_idx, "topk_idx", _I32, T * K), T, _ptr(expert_off, "expert_off", _I32, E + 1),
            _ptr(perm, "perm", _I32, T * K), _ptr(inv, "inv", _I32, T * K))
    d = desc.c()
    ws = _scratch(desc, T, topk_idx.device, stream) if ws is None else ws
    check(lib().moe_permute(C.byref(d), *args, _ws(ws), ws.numel(), _stream(stream)))


def expert_ffn(desc, layer, x, topk_idx, topk_w, shared_gate, y, ws=None, stream=None):
    T = _tokens(x, desc)
    K, H = desc.top_k, desc.hidden
    args = (_ptr(x), T, _ptr(topk_idx, "topk_idx", _I32, T * K), _ptr(topk_w, "topk_w", _F32, T * K),
            _ptr(shared_gate, "shared_gate", _F32, T), _ptr(y, "y", _F32, T * H))
    d, w = desc.c(), layer.c()
    ws = _scratch(desc, T, x.device, stream) if ws is None else ws
    check(lib().moe_expert_ffn(C.byref(d), C.byref(w), *args, _ws(ws), ws.numel(), _stream(stream)))


def layer_forward(desc, layer, x, y, topk_idx=None, topk_w=None, shared_gate=None, ws=None, stream=None):
    T = _tokens(x, desc)
    K, H = desc.top_k, desc.hidden
    args = (_ptr(x), T, _ptr(y, "y", _F32, T * H), _ptr(topk_idx, "topk_idx", _I32, T * K),
            _ptr(topk_w, "topk_w", _F32, T * K), _ptr(shared_gate, "shared_gate", _F32, T))
    d, w = desc.c(), layer.c()
    ws = _scratch(desc, T, x.device, stream) if ws is None else ws
    check(lib().moe_layer_forward(C.byref(d), C.byref(w), *args, _ws(ws), ws.numel(), _stream(stream)))


def layer_forward_static(desc, layer, x, y, topk_idx=None, topk_w=None, shared_gate=None, stream=None):
    """moe_layer_forward_static: the layer call with the library's static
    device scratch instead of a workspace (no allocation anywhere)."""
    T = _tokens(x, desc)
    K, H = desc.top_k, desc.hidden
    args = (_ptr(x), T, _ptr(y, "y", _F32, T * H), _ptr(topk_idx, "topk_idx", _I32, T * K),
            _ptr(topk_w, "topk_w", _F32, T * K), _ptr(shared_gate, "shared_gate", _F32, T))
    d, w = desc.c(), layer.c()
    check(lib().moe_layer_forward_static(C.byref(d), C.byref(w), *args, _stream(stream)))


def stack_epilogue(desc, y, r, x_next, stream=None):
    T, H = y.shape[0], desc.hidden
    args = (T, _ptr(y, "y", _F32, T * H), _ptr(r, "r", _F32, T * H), _ptr(x_next, "x_next", _ACT_DTYPES, T * H))
    d = desc.c()
    check(lib().moe_stack_epilogue(C.byref(d), *args, _stream(stream)))


def _layer_array(layers):
    arr = (LayerWeights * len(layers))(*[l.c() for l in layers])
    return arr


def _stack_args(desc, n_layers, x0, r, x_buf, ws, x_all, y_all, idx_all, w_all, gamma_all):
    T = _tokens(x0, desc, "x0")
    L, K, H = n_layers, desc.top_k, desc.hidden
    return (_ptr(x0), T, _ptr(r, "r", _F32, T * H), _ptr(x_buf, "x_buf", _ACT_DTYPES, T * H),
            _ptr(x_all, "x_all", _ACT_DTYPES, L * T * H), _ptr(y_all, "y_all", _F32, L * T * H),
            _ptr(idx_all, "idx_all", _I32, L * T * K), _ptr(w_all, "w_all", _F32, L * T * K),
            _ptr(gamma_all, "gamma_all", _F32, L * T), _ws(ws), ws.numel())


def stack_forward(desc, layers, x0, r, x_buf, ws, x_all=None, y_all=None, idx_all=None, w_all=None,
                  gamma_all=None, stream=None):
    args = _stack_args(desc, len(layers), x0, r, x_buf, ws, x_all, y_all, idx_all, w_all, gamma_all)
    d = desc.c()
    arr = _layer_array(layers)
    check(lib().moe_stack_forward(C.byref(d), arr, len(layers), *args, _stream(stream)))


class StackGraph:
    """moe_stack_forward captured once into a HIP graph; launch() replays it."""

    def __init__(self, desc, layers, x0, r, x_buf, ws, capture_stream, x_all=None, y_all=None, idx_all=None,
                 w_all=None, gamma_all=None):
        self._h = None
        args = _stack_args(desc, len(layers), x0, r, x_buf, ws, x_all, y_all, idx_all, w_all, gamma_all)
        d = desc.c()
        arr = _layer_array(layers)
        h = C.c_void_p()
        self._keep = (layers, x0, r, x_buf, ws, x_all, y_all, idx_all, w_all, gamma_all)
        check(lib().moe_stack_graph_create(C.byref(d), arr, len(layers), *args, _stream(capture_stream),
                                           C.byref(h)))
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
    H, K, L = desc.hidden, desc.top_k, len(layers)
    if idx_log is not None and (not isinstance(idx_log, np.ndarray) or idx_log.dtype != np.int32
                                or idx_log.size != L * 2 * K or not idx_log.flags.c_contiguous):
        raise ValueError(f"idx_log must be a contiguous int32 numpy array of {L * 2 * K} elements")
    args = (_ptr(x0, "x0", _ACT_DTYPES, H), _ptr(r, "r", _F32, H), _ptr(x_buf, "x_buf", _ACT_DTYPES, 2 * H),
            _ptr(idx_host, "idx_host", _I32, 2 * K, host=True))
    if isinstance(idx_host, torch.Tensor) and not idx_host.is_pinned():
        raise ValueError("idx_host must be pinned host memory")
    d = desc.c()
    arr = _layer_array(layers)
    log = None if idx_log is None else idx_log.ctypes.data
    check(lib().moe_pool_decode_step(C.byref(d), arr, L, pool._h, step, *args, log, int(pregate), _ws(ws),
                                     ws.numel(), _stream(stream)))


class DevPool:
    """GPU-resident slot pool (moe_devpool_*): the policy runs on the device,
    its state lives in a device tensor owned by this object."""

    def __init__(self, n_layers, n_experts, slots, aging_period, blob_stride, blob_bytes_, host_blobs, device_slab,
                 device_offsets, stream=None):
        if not isinstance(host_blobs, torch.Tensor) or not host_blobs.is_pinned():
            raise ValueError("host_blobs must be a pinned host tensor")
        cfg = SlotPoolConfig(n_layers, n_experts, slots, aging_period, blob_stride, blob_bytes_,
                             _ptr(host_blobs, "host_blobs", (torch.uint8,), host=True),
                             _ptr(device_slab, "device_slab", (torch.uint8,)),
                             _ptr(device_offsets, "device_offsets", (torch.int64,)), None, 0)
        n = C.c_size_t(0)
        check(lib().moe_devpool_state_bytes(C.byref(cfg), C.byref(n)))
        self.state = torch.empty(int(n.value), dtype=torch.uint8, device=device_slab.device)
        h = C.c_void_p()
        check(lib().moe_devpool_create(C.byref(cfg), _ptr(self.state), self.state.numel(), C.byref(h)))
        self._h = h
        self._keep = (host_blobs, device_slab, device_offsets)
        self.n_layers, self.n_experts, self.slots = n_layers, n_experts, slots
        self.reset(stream)

    def reset(self, stream=None):
        check(lib().moe_devpool_reset(self._h, _stream(stream)))

    def acquire(self, layer, experts, bump_step=False, trace=None, stream=None):
        """experts: device int32 tensor of ids; trace: device int32 [n, 3] or None."""
        n = experts.numel()
        check(lib().moe_devpool_acquire(self._h, layer, _ptr(experts, "experts", _I32, n), n, int(bump_step),
                                        _ptr(trace, "trace", _I32, 3 * n), _stream(stream)))

    def stats(self, stream=None):
        s = SlotPoolStats()
        step = C.c_uint64(0)
        err = C.c_int32(0)
        check(lib().moe_devpool_stats(self._h, C.byref(s), C.byref(step), C.byref(err), _stream(stream)))
        return dict(hits=s.hits, misses=s.misses, evictions=s.evictions, bytes_h2d=s.bytes_h2d,
                    prefetches=s.prefetches, step=step.value, error=err.value)

    def close(self):
        if self._h:
            lib().moe_devpool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _devpool_args(desc, layers, x0, r, x_buf, trace, ws):
    H, K, L = desc.hidden, desc.top_k, len(layers)
    return (_ptr(x0, "x0", _ACT_DTYPES, H), _ptr(r, "r", _F32, H), _ptr(x_buf, "x_buf", _ACT_DTYPES, 2 * H),
            _ptr(trace, "trace", _I32, L * K * 3), _ws(ws), ws.numel())


def pool_decode_step_dev(desc, layers, pool, x0, r, x_buf, ws, trace=None, stream=None):
    """One batch-1 token streamed through a DevPool (moe_pool_decode_step_dev):
    no host synchronisation; the pool's step advances on the device."""
    args = _devpool_args(desc, layers, x0, r, x_buf, trace, ws)
    d = desc.c()
    arr = _layer_array(layers)
    check(lib().moe_pool_decode_step_dev(C.byref(d), arr, len(layers), pool._h, *args, _stream(stream)))


class PoolGraph:
    """pool_decode_step_dev captured once (moe_pool_graph_create); every
    launch() runs the next token."""

    def __init__(self, desc, layers, pool, x0, r, x_buf, ws, capture_stream, trace=None):
        self._h = None
        args = _devpool_args(desc, layers, x0, r, x_buf, trace, ws)
        d = desc.c()
        arr = _layer_array(layers)
        h = C.c_void_p()
        self._keep = (layers, pool, x0, r, x_buf, ws, trace)
        check(lib().moe_pool_graph_create(C.byref(d), arr, len(layers), pool._h, *args, _stream(capture_stream),
                                          C.byref(h)))
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
        if isinstance(host_blobs, torch.Tensor) and not host_only and not host_blobs.is_pinned():
            raise ValueError("host_blobs must be pinned host memory")
        cfg = SlotPoolConfig(n_layers, n_experts, slots, aging_period, blob_stride, blob_bytes_,
                             _ptr(host_blobs, "host_blobs", (torch.uint8,), host=True),
                             _ptr(device_slab, "device_slab", (torch.uint8,)),
                             _ptr(device_offsets, "device_offsets", (torch.int64,)),
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
