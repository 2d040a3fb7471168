"""Workspace placement for prefill.

The attention kernel copies the K/V tile images from the workspace into LDS
with a hand-formed 64-bit scalar base address.  A workspace whose addresses
cross a point where the low 32 bits reach 2^31 (so that part of its tiles have
bit 31 of the low word set, the case a sign-extended low word would corrupt)
must give output bit-identical to the same call with an ordinary workspace:
head widths 128 (persistent local grid, and a global layer) and 64.
"""
import pytest
import torch

import global_muse_rope_amd as ma
from synth.workloads import glimmer, spark
from gpu_helpers import prefill_inputs_device

pytestmark = pytest.mark.gpu


def _straddling_workspace(need, dev):
    """A `need`-byte slice of a buffer over 4 GiB, 256-byte aligned, whose
    addresses run across a point with low 32 bits equal to 2^31."""
    big = torch.empty((1 << 32) + 2 * need + 4096, dtype=torch.uint8, device=dev)
    base = big.data_ptr()
    target = ((base >> 32) << 32) + (1 << 31)
    while target - need // 2 - 256 < base:
        target += 1 << 32
    off = target - need // 2 - base
    off -= off % 256
    assert 0 <= off and off + need <= big.numel()
    ws = big[off:off + need]
    lo = ws.data_ptr() & 0xFFFFFFFF
    last = (ws.data_ptr() + need - 1) & 0xFFFFFFFF
    assert lo < (1 << 31) <= last, (hex(ws.data_ptr()), need)
    return big, ws


@pytest.mark.parametrize("layer,T", [(glimmer(2048, 10000.0), 4096), (glimmer(0, 0.0), 2048),
                                     (spark(2048, 10000.0), 2048)])
def test_prefill_workspace_across_bit31(layer, T):
    dev = torch.device("cuda")
    print(f"prefill workspace across 2^31: {layer} T={T}", flush=True)
    x = prefill_inputs_device(layer, 1, T, seed=3)
    lp = ma.LayerParams.from_layer(layer)
    need = ma.prefill_workspace_size(lp, 1, T)
    ref = ma.prefill(lp, x["q"], x["k"], x["v"], x["g"])
    big, ws = _straddling_workspace(need, dev)
    y = ma.prefill(lp, x["q"], x["k"], x["v"], x["g"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
    del big, ws
    torch.cuda.empty_cache()
