"""The Python binding checks every auxiliary tensor before it reaches the
library: element type, element count and device.  A wrong count or a host
tensor would hand a kernel too few entries or a host pointer.  These run on
the CPU: the checks raise before any library call."""
import pytest
import torch

import global_muse_rope_amd as ma

CUDA0 = torch.device("cuda", 0)


def test_aux_dtype_count_and_device():
    pos = torch.zeros(12, dtype=torch.int32)
    with pytest.raises(TypeError):
        ma._check_aux("positions", pos.to(torch.int64), torch.int32, 12, CUDA0)
    with pytest.raises(ValueError, match="12 entries"):
        ma._check_aux("positions", torch.zeros(4, dtype=torch.int32), torch.int32, 12, CUDA0)
    with pytest.raises(ValueError, match="device tensor"):
        ma._check_aux("positions", pos, torch.int32, 12, CUDA0)


def test_workspace_checks():
    with pytest.raises(ValueError, match="device tensor"):
        ma._check_workspace(torch.empty(64, dtype=torch.uint8), 16, CUDA0)
    with pytest.raises(TypeError):
        ma._check_workspace(torch.empty(64, dtype=torch.float32), 16, CUDA0)


def test_cache_checks_host_tensors():
    k = torch.zeros((2, 1, 64, 64), dtype=torch.bfloat16)
    v = torch.zeros((2, 1, 64, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="cache.k"):
        ma._check_cache(ma.KvCache.ring(k, v), CUDA0)


def test_entry_points_reject_host_tensors():
    layer = ma.LayerParams(8, 2, 64, 0, 0.0, 1.0)
    q = torch.zeros((1, 4, 8, 64), dtype=torch.bfloat16)
    k = torch.zeros((1, 4, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        ma.prefill(layer, q, k, k, q)
    with pytest.raises(ValueError, match="device tensor"):
        ma.rope_qknorm(layer, q[0], k[0])
    with pytest.raises(ValueError, match="device tensor"):
        ma.decode(layer, q[0], k[0], k[0], q[0], torch.ones(1, dtype=torch.int32), 4,
                  ma.KvCache.ring(torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16),
                                  torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16)))


def test_block_output_and_weight_checks():
    """The block calls' out must match x (a wrong shape would be written past
    its end) and every weight must hold the layer's element count in its
    element type on the call's device."""
    layer = ma.LayerParams(8, 2, 64, 0, 0.0, 1.0)
    h = 256
    x = torch.zeros((1, 4, h), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out must be"):
        ma._check_block_out(torch.zeros((1, 3, h), dtype=torch.bfloat16), x)
    with pytest.raises(ValueError, match="out must be"):
        ma._check_block_out(torch.zeros((1, 4, h), dtype=torch.float32), x)
    with pytest.raises(ValueError, match="out must be"):
        ma._check_block_out(torch.zeros((1, h, 4), dtype=torch.bfloat16).transpose(1, 2), x)
    ma._check_block_out(torch.zeros((1, 4, h), dtype=torch.bfloat16), x)
    n = (2 * 8 + 2 * 2) * 64
    good = dict(in_norm=torch.zeros(h, dtype=torch.bfloat16), w_qkvg=torch.zeros((n, h), dtype=torch.bfloat16),
                w_o=torch.zeros((h, 8 * 64), dtype=torch.bfloat16), residual_gate=torch.zeros(h))
    cpu = torch.device("cpu")
    ma._check_block_weights(layer, ma.BlockWeights(**good), cpu)
    with pytest.raises(ValueError, match="w_qkvg"):
        ma._check_block_weights(layer, ma.BlockWeights(**dict(good, w_qkvg=torch.zeros((n - 64, h),
                                                                                          dtype=torch.bfloat16))), cpu)
    with pytest.raises(ValueError, match="residual_gate"):
        ma._check_block_weights(layer, ma.BlockWeights(**dict(good, residual_gate=torch.zeros(
            h, dtype=torch.bfloat16))), cpu)
    with pytest.raises(ValueError, match="in_norm"):
        ma._check_block_weights(layer, ma.BlockWeights(**good), CUDA0)
