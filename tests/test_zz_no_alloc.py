"""The allocation-free decode entry point (muse_attn_decode_noalloc) against
the workspace entry point (muse_attn_decode) on the same inputs, through the
C ABI: two calls in a row, the second with a smaller input, each within the
floating-point bar of the existing entry point's output (the two share the
launch plan and kernels, so they agree bit for bit) and of the fp64 oracle.
A call whose scratch need exceeds the fixed array is rejected before any
launch."""
import numpy as np
import pytest
import torch

import global_muse_rope_amd as ma
import oracle
import synth
from synth.workloads import Layer, SPARK_SCALE
from gpu_helpers import TOL, to_dev, max_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(kind, lens, seed):
    from test_gpu_parity import make_cache
    layer = Layer(hq=16, hkv=2, d=64, window=256 if kind == "ring" else 0, theta=10000.0 if kind == "ring" else 0.0,
                  scale=SPARK_SCALE, out_norm=True, out_eps=1e-6)
    B = len(lens)
    lens = np.array(lens, dtype=np.int32)
    cache, hk, hv = make_cache(kind, layer, B, lens, page_tokens=32, seed=seed)
    new = {n: synth.normal_bf16_bits(seed, sid, shp) for n, sid, shp in
           [("q", 12, (B, 16, 64)), ("k", 13, (B, 2, 64)), ("v", 14, (B, 2, 64)), ("g", 15, (B, 16, 64))]}
    return layer, lens, cache, hk, hv, new


@pytest.mark.parametrize("kind", ["paged", "ring"])
def test_noalloc_decode_matches_workspace_entry(kind):
    for call, lens in enumerate(([3000, 77, 1, 1500, 2600, 40], [200, 9, 120])):   # the second call is smaller
        layer, lens, cache, hk, hv, new = _case(kind, lens, seed=4 + call)
        dn = {n: to_dev(b) for n, b in new.items()}
        kv = torch.from_numpy(lens).to(DEV)
        lp = ma.LayerParams.from_layer(layer)
        maxl = int(lens.max())
        y_ws = ma.decode(lp, dn["q"], dn["k"], dn["v"], dn["g"], kv, maxl, cache)
        y_na = ma.decode_noalloc(lp, dn["q"], dn["k"], dn["v"], dn["g"], kv, maxl, cache)
        torch.cuda.synchronize()
        a, b = y_ws.float().cpu().numpy(), y_na.float().cpu().numpy()
        diff = max_err(b, a)
        worst = 0.0
        for i in range(len(lens)):
            L = int(lens[i])
            fb = {n: synth.bf16_bits_to_f64(v)[i] for n, v in new.items()}
            ref = oracle.decode_one(fb["q"], fb["k"], fb["v"], fb["g"], hk[i, :max(L - 1, 0)].astype(np.float64),
                                    hv[i, :max(L - 1, 0)].astype(np.float64), 0, L, layer)
            worst = max(worst, max_err(b[i], ref))
        print(f"noalloc {kind} call {call} lens {lens.tolist()}: |noalloc - decode| = {diff:.3e}, "
              f"vs oracle {worst:.3e}, bit-identical {torch.equal(y_ws, y_na)}", flush=True)
        assert diff <= TOL and worst <= TOL


def test_noalloc_rejects_calls_beyond_its_scratch():
    layer = Layer(hq=128, hkv=16, d=64, window=0, theta=0.0, scale=SPARK_SCALE, out_norm=True, out_eps=1e-6)
    lp = ma.LayerParams.from_layer(layer)
    B, maxl, pt = 64, 1 << 20, 32
    cache = ma.KvCache.paged(torch.zeros((4, 16, pt, 64), dtype=torch.bfloat16, device=DEV),
                             torch.zeros((4, 16, 64, pt), dtype=torch.bfloat16, device=DEV),
                             torch.zeros((B, maxl // pt), dtype=torch.int32, device=DEV), pt)
    assert ma.decode_workspace_size(lp, B, maxl, cache) > (80 << 20)
    q = torch.zeros((B, 128, 64), dtype=torch.bfloat16, device=DEV)
    kv = torch.ones((B, 16, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ma.MuseError, match="scratch"):
        ma.decode_noalloc(lp, q, kv, kv, q, torch.ones(B, dtype=torch.int32, device=DEV), maxl, cache)
