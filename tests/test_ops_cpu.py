"""The torch binding's own checks (no GPU needed)."""

import pytest
import torch

from attention_int8_quantized_amd import ops


def test_output_tensors_are_checked_before_any_call():
    made = ops._out(None, (2, 3), torch.float32, "cpu")
    assert made.shape == (2, 3) and made.dtype == torch.float32
    with pytest.raises(ValueError):
        ops._out(torch.empty(6), (2, 3), torch.float32, "cpu")        # not a GPU tensor


def test_workspace_must_be_a_gpu_tensor():
    with pytest.raises(ValueError):
        ops._nbytes(torch.empty(16, dtype=torch.uint8))


def test_cache_inputs_must_be_gpu_tensors():
    q = torch.zeros(1, 4, 64)
    kc = torch.zeros(1, 8, 64, dtype=torch.int8)
    ks = torch.zeros(1, 8, 2, dtype=torch.float16)
    with pytest.raises(ValueError):
        ops.verify(q, kc, ks, kc, ks, ctx_len=4)
    with pytest.raises(ValueError):
        ops.stream_read(torch.zeros(16))
