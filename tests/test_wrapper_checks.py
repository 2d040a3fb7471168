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
