"""GPU parity of int8 affine experts (the pages' other group-quantisation
width) against the fp64 oracle, through the C ABI, on both kernel families:
the per-row GEMVs and the grouped matrix-core kernels (bytes enter the
matrix cores as exact fp16 subnormals)."""
import dataclasses

import numpy as np
import pytest

import synth
from moe_testlib import DeviceLayer
from test_gpu_layer import RAGGED, check_layer

pytestmark = pytest.mark.gpu

TINY8 = dataclasses.replace(synth.TINY, name="tiny_i8", bits=8, scale_lo=1e-4, scale_hi=1e-3, weight_seed=21,
                            token_seed=121)
RAGGED8 = dataclasses.replace(RAGGED, name="ragged_i8", bits=8, scale_lo=1e-4, scale_hi=1e-3, weight_seed=22,
                              token_seed=122)
TINY8_G128 = dataclasses.replace(TINY8, name="tiny_i8_g128", inter=128, shared_inter=128, group=128,
                                 act_dtype="bf16", weight_seed=23, token_seed=123)
BAT80I8 = dataclasses.replace(synth.BAT80, name="bat80i8", bits=8, scale_lo=1e-4, scale_hi=1e-3)


@pytest.mark.parametrize("path", [0, 1, 2], ids=["auto", "gemv", "grouped"])
def test_tiny_int8(path):
    check_layer(TINY8, path, gpu_fill=False)


@pytest.mark.parametrize("path", [0, 1, 2], ids=["auto", "gemv", "grouped"])
def test_ragged_int8(path):
    check_layer(RAGGED8, path, gpu_fill=False)


@pytest.mark.parametrize("path", [1, 2], ids=["gemv", "grouped"])
def test_int8_general_affine_bias(path):
    check_layer(RAGGED8, path, general_bias_seed=9)


@pytest.mark.parametrize("path", [1, 2], ids=["gemv", "grouped"])
def test_int8_group_128_no_shared(path):
    check_layer(TINY8_G128, path, gpu_fill=False)
    check_layer(TINY8_G128, path, shared=False, gpu_fill=False)


def test_int8_grouped_group_32_many_tokens():
    # group 32 (two groups per 64-column chunk) with units of up to 16 tokens
    wl = dataclasses.replace(TINY8, name="tiny_i8_many", tokens=40, zipf_s=1.2, weight_seed=24, token_seed=124)
    check_layer(wl, 2, gpu_fill=False)
    check_layer(wl, 0, general_bias_seed=3)


def test_int8_gpu_fill_matches_host_packer():
    import torch
    from int4_routed_expert_router_amd import api
    for wl, experts in ((TINY8, [0, 9, 15]), (synth.DEC80I8, [0, 401]), (RAGGED8, [23])):
        stride = api.blob_bytes(wl.hidden, wl.inter, wl.group, 8)
        dev = torch.empty(stride * len(experts), dtype=torch.uint8, device="cuda")
        for k, e in enumerate(experts):
            api.synth_fill_experts(wl.weight_seed, 2, e, 1, wl.hidden, wl.inter, wl.group, wl.scale_lo, wl.scale_hi,
                                   dev[k * stride:], stride, bits=8)
        got = dev.cpu().numpy()
        for k, e in enumerate(experts):
            want = api.pack_expert(synth.expert_raw(wl, 2, e), wl.hidden, wl.inter, wl.group, 8)
            assert np.array_equal(got[k * stride:(k + 1) * stride], want), (wl.name, e)


@pytest.mark.parametrize("layer", [0, 47])
def test_int8_decode_layer_full_size(layer):
    worst, tol, flagged = check_layer(synth.DEC80I8, 0, layer=layer)
    print(f"dec80i8 layer {layer}: max err {worst:.3e} (tol {tol:.3e}), near ties {flagged}")


@pytest.mark.parametrize("path", [0, 1], ids=["auto_grouped", "gemv"])
def test_int8_batched_layer_full_size(path):
    # 64 tokens x (10 + 1) rows: AUTO takes the grouped family
    worst, tol, flagged = check_layer(BAT80I8, path, layer=3)
    print(f"bat80i8 path {path}: max err {worst:.3e} (tol {tol:.3e}), near ties {flagged}")


def test_int8_and_int4_blobs_differ_in_stride():
    # the descriptor's width decides the stride check: an int4-sized stride is
    # too small for int8 blobs
    import torch
    from int4_routed_expert_router_amd import api, MoeError
    dl = DeviceLayer(TINY8, 0, use_gpu_fill=True)
    d8 = api.Desc(TINY8.hidden, TINY8.n_experts, TINY8.top_k, TINY8.inter, TINY8.shared_inter, TINY8.group, "f16",
                  1, 8)
    small = api.Layer(dl.router_w, dl.router_bias, dl.experts, api.blob_bytes(TINY8.hidden, TINY8.inter, TINY8.group),
                      None, dl.shared)
    x = torch.zeros(2, TINY8.hidden, dtype=torch.int16, device="cuda")
    y = torch.empty(2, TINY8.hidden, dtype=torch.float32, device="cuda")
    with pytest.raises(MoeError, match="MOE_EINVAL"):
        api.layer_forward(d8, small, x, y)
