"""ctypes declarations of the C ABI (include/moe.h, include/moe_synth.h,
include/moe_slotpool.h).  Loading fails loudly when the library is missing:
there is no fallback path."""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_amd.so")

MOE_OK, MOE_EINVAL, MOE_ESHAPE, MOE_EWORKSPACE, MOE_EHIP, MOE_EPOOLFULL, MOE_EBUSY, MOE_ENOMEM = 0, -1, -2, -3, -4, -5, -6, -7
MOE_F16, MOE_BF16 = 1, 2
MOE_PATH_AUTO, MOE_PATH_GEMV, MOE_PATH_GROUPED = 0, 1, 2
MOE_GEMV_MAX_ROWS = 32
MOE_POOL_HOST_ONLY = 1
MOE_POOL_DMA_COPY = 2
MOE_TIME_GATEUP, MOE_TIME_DOWN, MOE_TIME_ROUTER = 0, 1, 2
MOE_FLAG_F16_RANGE = 1
MOE_FLAG_STREAM_WAIT = 2

STATUS_NAMES = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_ESHAPE", -3: "MOE_EWORKSPACE", -4: "MOE_EHIP",
                -5: "MOE_EPOOLFULL", -6: "MOE_EBUSY", -7: "MOE_ENOMEM"}


class LayerDesc(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32), ("inter", C.c_int32),
                ("shared_inter", C.c_int32), ("group_size", C.c_int32), ("act_dtype", C.c_int32),
                ("path", C.c_int32), ("weight_bits", C.c_int32)]


class LayerWeights(C.Structure):
    _fields_ = [("router_w", C.c_void_p), ("router_bias", C.c_void_p), ("experts", C.c_void_p),
                ("expert_stride", C.c_uint64), ("expert_offset", C.c_void_p), ("shared", C.c_void_p)]


class GdnDesc(C.Structure):
    _fields_ = [("batch", C.c_int32), ("k_heads", C.c_int32), ("v_heads", C.c_int32), ("head_k_dim", C.c_int32),
                ("head_v_dim", C.c_int32), ("act_dtype", C.c_int32)]


class SlotPoolConfig(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("n_experts", C.c_int32), ("slots_per_layer", C.c_int32),
                ("aging_period", C.c_int32), ("blob_stride", C.c_uint64), ("blob_bytes", C.c_uint64),
                ("host_blobs", C.c_void_p), ("device_slab", C.c_void_p), ("device_offsets", C.c_void_p),
                ("copy_stream", C.c_void_p), ("flags", C.c_uint32)]


class SlotPoolStats(C.Structure):
    _fields_ = [("hits", C.c_uint64), ("misses", C.c_uint64), ("evictions", C.c_uint64), ("bytes_h2d", C.c_uint64),
                ("prefetches", C.c_uint64)]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None

vp, i32, u64, f32 = C.c_void_p, C.c_int32, C.c_uint64, C.c_float
PROTOS = {
    "moe_last_error": (C.c_char_p, []),
    "moe_version": (C.c_char_p, []),
    "moe_blob_bytes": (u64, [i32, i32, i32]),
    "moe_pack_expert": (i32, [i32, i32, i32] + [vp] * 10),
    "moe_blob_bytes_q": (u64, [i32, i32, i32, i32]),
    "moe_pack_expert_q": (i32, [i32, i32, i32, i32] + [vp] * 10),
    "moe_workspace_bytes": (i32, [vp, i32, C.POINTER(C.c_size_t)]),
    "moe_workspace_status": (i32, [vp, i32, C.POINTER(C.c_size_t)]),
    "moe_route": (i32, [vp, vp, vp, i32, vp, vp, vp, vp, vp, C.c_size_t, vp]),
    "moe_permute": (i32, [vp, vp, i32, vp, vp, vp, vp, C.c_size_t, vp]),
    "moe_expert_ffn": (i32, [vp, vp, vp, i32, vp, vp, vp, vp, vp, C.c_size_t, vp]),
    "moe_layer_forward": (i32, [vp, vp, vp, i32, vp, vp, vp, vp, vp, C.c_size_t, vp]),
    "moe_layer_forward_static": (i32, [vp, vp, vp, i32, vp, vp, vp, vp, vp]),
    "moe_stack_epilogue": (i32, [vp, i32, vp, vp, vp, vp]),
    "moe_stack_forward": (i32, [vp, vp, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp]),
    "moe_stack_graph_create": (i32, [vp, vp, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp,
                                     C.POINTER(vp)]),
    "moe_graph_launch": (i32, [vp, vp]),
    "moe_stack_set_kernel_events": (i32, [vp, vp, i32, i32]),
    "moe_graph_destroy": (None, [vp]),
    "moe_synth_fill_experts": (i32, [u64, i32, i32, i32, i32, i32, i32, i32, f32, f32, vp, u64, vp]),
    "moe_synth_philox": (i32, [vp, vp, vp, i32, vp]),
    "moe_gdn_step": (i32, [C.POINTER(GdnDesc), vp, vp, vp, vp, vp, f32, vp, vp, vp]),
    "slotpool_create": (i32, [C.POINTER(SlotPoolConfig), C.POINTER(vp)]),
    "slotpool_acquire": (i32, [vp, i32, vp, i32, u64, vp, vp, vp, vp]),
    "slotpool_prefetch": (i32, [vp, i32, vp, i32, u64, vp, vp, vp, vp, vp]),
    "slotpool_release": (i32, [vp, i32, vp]),
    "slotpool_evict": (i32, [vp, i32, i32]),
    "slotpool_stats": (i32, [vp, C.POINTER(SlotPoolStats)]),
    "slotpool_destroy": (None, [vp]),
    "slotpool_get_config": (i32, [vp, C.POINTER(SlotPoolConfig)]),
    "moe_read_probe": (i32, [vp, u64, i32, vp, vp]),
    "moe_devpool_state_bytes": (i32, [C.POINTER(SlotPoolConfig), C.POINTER(C.c_size_t)]),
    "moe_devpool_create": (i32, [C.POINTER(SlotPoolConfig), vp, C.c_size_t, C.POINTER(vp)]),
    "moe_devpool_reset": (i32, [vp, vp]),
    "moe_devpool_acquire": (i32, [vp, i32, vp, i32, i32, vp, vp]),
    "moe_devpool_stats": (i32, [vp, C.POINTER(SlotPoolStats), C.POINTER(u64), C.POINTER(i32), vp]),
    "moe_devpool_destroy": (None, [vp]),
    "moe_pool_decode_step_dev": (i32, [vp, vp, i32, vp, vp, vp, vp, vp, vp, C.c_size_t, vp]),
    "moe_pool_graph_create": (i32, [vp, vp, i32, vp, vp, vp, vp, vp, vp, C.c_size_t, vp, C.POINTER(vp)]),
    "moe_pool_decode_step": (i32, [vp, vp, i32, vp, u64, vp, vp, vp, vp, vp, i32, vp, C.c_size_t, vp]),
}


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               f"`python -m int4_routed_expert_router_amd.build` (no fallback path exists)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in PROTOS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())
