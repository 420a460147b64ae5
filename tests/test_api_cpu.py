"""The Python binding refuses arguments the C ABI would dereference in the
wrong memory (host tensors where device addresses are read, unpinned host
memory for asynchronous copies), non-contiguous or wrongly sized tensors, and
temporary workspaces it cannot keep alive on a raw stream handle.  Every
refusal happens before any call into the library or any GPU work."""
import numpy as np
import pytest
import torch

from int4_routed_expert_router_amd import api

DESC = api.Desc(256, 16, 2, 64, 64, 32, "f16")


def cpu_layer():
    return api.Layer(4096, None, 4096, api.blob_bytes(256, 64, 32), None, 4096)


def test_host_tensor_as_device_argument_is_refused():
    x = torch.zeros(4, 256, dtype=torch.int16)
    y = torch.zeros(4, 256, dtype=torch.float32)
    with pytest.raises(ValueError, match="x must be a CUDA tensor"):
        api.layer_forward(DESC, cpu_layer(), x, y, ws=4096)
    with pytest.raises(ValueError, match="must be a CUDA tensor"):
        api.Layer(torch.zeros(17, 256, dtype=torch.int16), None, 4096, 30720).c()


def test_wrong_dtype_size_and_layout_are_refused():
    t = torch.zeros(8, 6, dtype=torch.float32)
    with pytest.raises(ValueError, match="contiguous"):
        api._ptr(t.t(), "y", host=True)
    with pytest.raises(ValueError, match="elements"):
        api._ptr(t, "y", (torch.float32,), 40, host=True)
    with pytest.raises(ValueError, match="dtype"):
        api._ptr(t, "idx", (torch.int32,), 48, host=True)
    assert api._ptr(t, "y", (torch.float32,), 48, host=True) == t.data_ptr()
    assert api._ptr(None) is None and api._ptr(1 << 20) == 1 << 20


def test_temporary_workspace_needs_a_torch_stream():
    with pytest.raises(ValueError, match="raw stream handle"):
        api._scratch(DESC, 4, "cpu", 12345)


def test_pool_decode_needs_pinned_index_buffer():
    host = torch.zeros(2, 2, dtype=torch.int32)          # not pinned
    with pytest.raises(ValueError, match="pinned"):
        api.pool_decode_step(DESC, [cpu_layer()], None, 0, 4096, 4096, 4096, host, 4096)
    with pytest.raises(ValueError, match="idx_log"):
        api.pool_decode_step(DESC, [cpu_layer()], None, 0, 4096, 4096, 4096, host, 4096,
                             idx_log=np.zeros((1, 2, 2), np.int64))
