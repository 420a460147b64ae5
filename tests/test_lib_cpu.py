"""CPU-side checks of the C ABI library: it loads, exports what the headers
declare, the host packer and the pool policy match the oracle, and argument
validation rejects bad calls before touching the GPU."""
import ctypes as C
import dataclasses
import os
import re

import numpy as np
import pytest

import synth
from oracle import blob_ref
from oracle.pool_sim import PoolFull, PoolSim

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from int4_routed_expert_router_amd import _lib as L
    return L


def header_symbols():
    syms = set()
    for name in os.listdir(os.path.join(ROOT, "include")):
        if name.endswith(".h"):
            text = open(os.path.join(ROOT, "include", name)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            for m in re.finditer(r"\b(moe_[a-z_0-9]+|slotpool_[a-z_]+)\s*\(", text):
                syms.add(m.group(1))
    return syms


def test_library_exports_every_declared_symbol():
    L = _lib()
    lib = L.lib()
    syms = header_symbols()
    assert len(syms) >= 20
    for s in sorted(syms):
        assert hasattr(lib, s), f"{s} declared in include/ but not exported"
    assert set(L.PROTOS) <= syms | {"moe_last_error", "moe_version"}


def test_blob_bytes_and_packer_match_oracle():
    from int4_routed_expert_router_amd import api
    assert api.blob_bytes(2048, 512, 64) == 1_769_472 == blob_ref.blob_bytes(2048, 512, 64)
    assert api.blob_bytes(100, 64, 32) == 0
    for wl in (synth.TINY, synth.DEC80):
        raw = synth.expert_raw(wl, 1, 2)
        got = api.pack_expert(raw, wl.hidden, wl.inter, wl.group)
        back = blob_ref.parse_blob(got, wl.hidden, wl.inter, wl.group)
        for name in raw:
            for a, b in zip(raw[name], back[name]):
                assert np.array_equal(a, b)


def test_int8_blob_bytes_and_packer_match_oracle():
    from int4_routed_expert_router_amd import api
    assert api.blob_bytes(2048, 512, 64, 8) == 3_342_336 == blob_ref.blob_bytes(2048, 512, 64, bits=8)
    assert api.blob_bytes(256, 64, 32, 6) == 0
    for wl in (synth.TINY, synth.DEC80I8):
        wl8 = wl if wl.bits == 8 else dataclasses.replace(wl, bits=8)
        raw = synth.expert_raw(wl8, 1, 2)
        got = api.pack_expert(raw, wl8.hidden, wl8.inter, wl8.group, 8)
        assert got.size == blob_ref.blob_bytes(wl8.hidden, wl8.inter, wl8.group, bits=8)
        back = blob_ref.parse_blob(got, wl8.hidden, wl8.inter, wl8.group, bits=8)
        for name in raw:
            for a, b in zip(raw[name], back[name]):
                assert np.array_equal(a, b)
        # the oracle's own writer gives the same bytes
        want = blob_ref.pack_blob(raw["gate"], raw["up"], raw["down"], wl8.hidden, wl8.inter, wl8.group, bits=8)
        assert np.array_equal(got, want)


def test_int8_desc_validation():
    from int4_routed_expert_router_amd import api, MoeError
    from int4_routed_expert_router_amd._lib import MOE_PATH_GEMV
    n8 = api.workspace_bytes(api.Desc(2048, 512, 10, 512, 512, 64, weight_bits=8), 64)
    assert n8 == api.workspace_bytes(api.Desc(2048, 512, 10, 512, 512, 64), 64)
    api.workspace_bytes(api.Desc(256, 16, 2, 64, 64, 32, path=MOE_PATH_GEMV, weight_bits=8), 4)
    api.workspace_bytes(api.Desc(256, 16, 2, 64, 64, 32, weight_bits=0), 4)   # 0 reads as int4
    with pytest.raises(MoeError, match="MOE_ESHAPE"):
        api.workspace_bytes(api.Desc(256, 16, 2, 64, 64, 32, weight_bits=6), 4)
    api.workspace_bytes(api.Desc(256, 16, 2, 64, 64, 32, path=2, weight_bits=8), 4)   # int8 on the matrix cores


def test_packer_rejects_bad_nibbles():
    from int4_routed_expert_router_amd import api, MoeError
    raw = synth.expert_raw(synth.TINY, 0, 0)
    q = raw["gate"][0].copy()
    q[3, 4] = 16
    raw["gate"] = (q, raw["gate"][1], raw["gate"][2])
    with pytest.raises(MoeError, match="MOE_EINVAL"):
        api.pack_expert(raw, 256, 64, 32)


def test_workspace_and_validation_errors():
    from int4_routed_expert_router_amd import api, MoeError
    from int4_routed_expert_router_amd._lib import LayerDesc, LayerWeights, lib
    d = api.Desc(2048, 512, 10, 512, 512, 64)
    n = api.workspace_bytes(d, 64)
    assert n > 64 * 11 * 2048 * 4
    assert api.workspace_bytes(d, 0) > 0
    bad = [api.Desc(100, 16, 2, 64, 64, 32), api.Desc(256, 16, 17, 64, 64, 32), api.Desc(256, 16, 2, 96, 64, 32),
           api.Desc(256, 16, 2, 64, 64, 48), api.Desc(256, 2000, 2, 64, 64, 32), api.Desc(256, 16, 2, 64, 32, 32)]
    for b in bad:
        with pytest.raises(MoeError, match="MOE_ESHAPE"):
            api.workspace_bytes(b, 4)
    with pytest.raises(MoeError, match="MOE_EINVAL"):
        api.workspace_bytes(api.Desc(256, 16, 2, 64, 64, 32, act_dtype="fp8"), 4)
    # layer call with NULL weights / misaligned pointers is rejected before any GPU work
    L = lib()
    dc = api.Desc(256, 16, 2, 64, 64, 32, "f16").c()
    w = LayerWeights(None, None, None, 0, None, None)
    st = L.moe_layer_forward(C.byref(dc), C.byref(w), 16, 4, 16, None, None, None, 256, 10 ** 6, None)
    assert st == -1 and b"router_w" in L.moe_last_error()
    w = LayerWeights(4096, None, 4096 + 8, 30720, None, 8192)
    st = L.moe_layer_forward(C.byref(dc), C.byref(w), 16, 4, 16, None, None, None, 256, 10 ** 6, None)
    assert st == -1 and b"experts" in L.moe_last_error()
    w = LayerWeights(4096, None, 8192, 30720, None, 8192)
    st = L.moe_layer_forward(C.byref(dc), C.byref(w), 16, 4, 16, None, None, None, 256, 16, None)
    assert st == -3 and b"workspace" in L.moe_last_error()
    # zero tokens is a no-op even with no buffers
    assert L.moe_layer_forward(C.byref(dc), C.byref(w), None, 0, None, None, None, None, None, 0, None) == 0
    assert L.moe_last_error() == b""
    # graph capture refuses the NULL stream
    h = C.c_void_p()
    st = L.moe_stack_graph_create(C.byref(dc), None, 0, None, 0, None, None, None, None, None, None, None, None, 0,
                                  None, C.byref(h))
    assert st == -1


def _pool_trace(seed, layers, experts, slots, period, steps, k):
    rng = np.random.default_rng(seed)
    perm = [rng.permutation(experts) for _ in range(layers)]
    for s in range(steps):
        if s and s % 17 == 0:
            perm = [rng.permutation(experts) for _ in range(layers)]
        for l in range(layers):
            p = 1.0 / (1.0 + perm[l]) ** 1.1
            p /= p.sum()
            yield s, l, rng.choice(experts, size=k, replace=False, p=p)


@pytest.mark.parametrize("seed,slots,period", [(1, 8, 4), (2, 3, 0), (3, 12, 1), (4, 5, 32)])
def test_pool_core_matches_oracle_simulator(seed, slots, period):
    from int4_routed_expert_router_amd import api
    layers, experts, k = 3, 24, 3
    pool = api.SlotPool(layers, experts, slots, period, blob_bytes_=100, host_only=True)
    sim = PoolSim(layers, experts, slots, period, blob_bytes=100)
    for s, l, ex in _pool_trace(seed, layers, experts, slots, period, 120, k):
        got = pool.acquire(l, ex, s, compute_stream=False)
        want = sim.acquire(l, ex, s)
        assert got == want, (s, l, ex)
        pool.release(l, compute_stream=False)
        sim.release(l)
        if s % 11 == 5:
            pool.evict(l, int(ex[0]))
            sim.evict(l, int(ex[0]))
    assert pool.stats() == sim.stats()


@pytest.mark.parametrize("seed,slots,period", [(5, 8, 4), (6, 4, 0), (7, 12, 2)])
def test_pool_prefetch_matches_oracle_simulator(seed, slots, period):
    # before each acquire, a prefetch of a prediction: the true set with one or
    # two entries replaced by random experts (as a pre-gated router would err)
    from int4_routed_expert_router_amd import api
    layers, experts, k = 3, 24, 4
    rng = np.random.default_rng(seed + 100)
    pool = api.SlotPool(layers, experts, slots, period, blob_bytes_=100, host_only=True)
    sim = PoolSim(layers, experts, slots, period, blob_bytes=100)
    for s, l, ex in _pool_trace(seed, layers, experts, slots, period, 100, k):
        if s % 5 != 4:   # some acquires come without a prefetch
            pred = list(ex)
            for j in rng.choice(k, size=int(rng.integers(0, 3)), replace=False):
                c = int(rng.integers(0, experts))
                if c not in pred:
                    pred[j] = c
            assert pool.prefetch(l, pred, s, compute_stream=False) == sim.prefetch(l, pred, s), (s, l, pred)
        assert pool.acquire(l, ex, s, compute_stream=False) == sim.acquire(l, ex, s), (s, l, ex)
        if s % 7 == 3:   # a prefetch while the layer is pinned may not take pinned slots
            other = [int(e) for e in rng.choice(experts, size=3, replace=False)]
            assert pool.prefetch(l, other, s, compute_stream=False) == sim.prefetch(l, other, s)
        pool.release(l, compute_stream=False)
        sim.release(l)
    assert pool.stats() == sim.stats()
    assert sim.stats()["prefetches"] > 0


def test_pool_error_paths():
    from int4_routed_expert_router_amd import api, MoeError
    pool = api.SlotPool(1, 6, 2, 4, host_only=True)
    sim = PoolSim(1, 6, 2, 4)
    assert pool.acquire(0, [0, 1], 0, False) == sim.acquire(0, [0, 1], 0)
    with pytest.raises(MoeError, match="MOE_EBUSY"):
        pool.evict(0, 1)
    with pytest.raises(MoeError, match="MOE_EPOOLFULL"):
        pool.acquire(0, [2], 1, False)
    with pytest.raises(PoolFull):
        sim.acquire(0, [2], 1)
    # prefetch never fails for lack of slots (both slots are pinned) but rejects bad ids
    assert pool.prefetch(0, [2, 3], 1, False) == sim.prefetch(0, [2, 3], 1) == []
    with pytest.raises(MoeError, match="MOE_EINVAL"):
        pool.prefetch(0, [4, 4], 1, False)
    with pytest.raises(MoeError, match="MOE_EINVAL"):
        pool.prefetch(0, [6], 1, False)
    with pytest.raises(MoeError, match="MOE_EINVAL"):
        pool.acquire(0, [3, 3], 1, False)
    with pytest.raises(MoeError, match="MOE_EINVAL"):
        pool.acquire(0, [6], 1, False)
    pool.release(0, False)
    sim.release(0)
    assert pool.acquire(0, [2], 1, False) == sim.acquire(0, [2], 1)
    assert pool.stats() == sim.stats()
    with pytest.raises(MoeError, match="MOE_ESHAPE"):
        api.SlotPool(1, 4, 5, 4, host_only=True)
    with pytest.raises(MoeError, match="MOE_EINVAL"):
        api.SlotPool(1, 8, 4, 4)               # device pool without buffers


def test_gdn_validation_before_any_gpu_work():
    import ctypes as C
    from int4_routed_expert_router_amd._lib import GdnDesc, lib, MOE_BF16
    L = lib()
    bad = [GdnDesc(4, 16, 32, 64, 128, MOE_BF16), GdnDesc(4, 16, 32, 128, 24, MOE_BF16),
           GdnDesc(4, 16, 24, 128, 128, MOE_BF16), GdnDesc(4, 16, 32, 128, 272, MOE_BF16),
           GdnDesc(-1, 16, 32, 128, 128, MOE_BF16), GdnDesc(70000, 16, 32, 128, 128, MOE_BF16)]
    for d in bad:
        assert L.moe_gdn_step(C.byref(d), None, None, None, None, None, 1.0, None, None, None) == -2
    d = GdnDesc(4, 16, 32, 128, 128, 7)
    assert L.moe_gdn_step(C.byref(d), None, None, None, None, None, 1.0, None, None, None) == -1
    d = GdnDesc(0, 16, 32, 128, 128, MOE_BF16)     # empty batch: no-op, no buffers needed
    assert L.moe_gdn_step(C.byref(d), None, None, None, None, None, 1.0, None, None, None) == 0
    d = GdnDesc(2, 16, 32, 128, 128, MOE_BF16)
    assert L.moe_gdn_step(C.byref(d), None, None, None, None, None, 1.0, None, None, None) == -1
    st = L.moe_gdn_step(C.byref(d), 4096, 4096, 4096, 4096, 4096, 1.0, 4100, 4096, None)
    assert st == -1 and b"aligned" in L.moe_last_error()


def test_pool_decode_validation_before_any_gpu_work():
    import ctypes as C
    from int4_routed_expert_router_amd import api
    from int4_routed_expert_router_amd._lib import lib
    L = lib()
    d = api.Desc(256, 16, 2, 64, 64, 32, "f16").c()
    arr = api._layer_array([api.Layer(4096, None, 4096, 30720, None, 4096)])
    host = np.zeros((2, 2), np.int32)
    args = (C.byref(d), arr, 1)
    tail = (0, 4096, 4096, 4096, host.ctypes.data, None, 0, 4096, 1 << 20, None)
    assert L.moe_pool_decode_step(*args, None, *tail) == -1 and b"pool" in L.moe_last_error()
    pool = api.SlotPool(1, 16, 4, 0, host_only=True)
    assert L.moe_pool_decode_step(*args, pool._h, *tail) == -1 and b"HOST_ONLY" in L.moe_last_error()
    st = L.moe_pool_decode_step(*args, pool._h, 0, 4096, 4096, 4096, host.ctypes.data, None, -1, 4096, 1 << 20,
                                None)
    assert st == -1 and b"pregate" in L.moe_last_error()
    pool.close()


def test_device_pool_state_size_and_validation():
    import ctypes as C
    from int4_routed_expert_router_amd._lib import SlotPoolConfig, lib
    L = lib()
    n = C.c_size_t(0)
    cfg = SlotPoolConfig(48, 512, 128, 32, 1769472, 1769472, None, None, None, None, 0)
    assert L.moe_devpool_state_bytes(C.byref(cfg), C.byref(n)) == 0
    # header, epochs, slot table, then per slot expert, count and last use, and the miss list
    assert n.value >= 48 * 512 * 4 + 48 * 128 * (4 + 4 + 8)
    bad = SlotPoolConfig(48, 512, 0, 32, 1769472, 1769472, None, None, None, None, 0)
    assert L.moe_devpool_state_bytes(C.byref(bad), C.byref(n)) == -2
    h = C.c_void_p()
    assert L.moe_devpool_create(C.byref(cfg), None, 0, C.byref(h)) == -1      # no host blobs / state
    big = SlotPoolConfig(1, 4096, 2048, 0, 256, 256, None, None, None, None, 0)
    assert L.moe_devpool_create(C.byref(big), None, 0, C.byref(h)) == -2      # more than 1024 slots
