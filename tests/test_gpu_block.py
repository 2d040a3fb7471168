"""GPU parity of the attention half of a decoder block (input norm,
projections through hipBLASLt, the layer, o_proj, post-norm and residual)
against the fp64 block oracle, through the C ABI.

Tolerance, derived from the arithmetic: the device rounds the q/k/v/gate
projections to bf16 (relative error up to 2^-9 per element) before the
layer, and the weightless QK-norm turns that into a logit error of about
s / sqrt(D) * sqrt(2 D / 3) * 2^-9 (standard deviation 0.009 for Spark, 0.006
for Glimmer), i.e. about 1 % in each softmax weight; normed output, gate and
o_proj carry it to an O(1) branch with a per-element standard deviation near
0.01, and the largest of 10^5-10^6 outputs lies near 5 sigma.  The other
roundings (h, o, the o_proj output, the stored result) add a few 2^-9.
BLOCK_TOL = 6e-2 bounds the max-abs error over a call.
"""
import numpy as np
import pytest
import torch

import global_muse_rope_amd as ma
import synth
from oracle import block as OB
from synth.workloads import Layer, GLIMMER_SCALE, SPARK_SCALE
from gpu_helpers import to_dev, max_err

pytestmark = pytest.mark.gpu
DEV = "cuda"
BLOCK_TOL = 6e-2


def _f(bits):
    return synth.bf16_bits_to_f64(bits)


def make_block(layer, hidden, spark, seed=0):
    """Seeded weights (bf16 bits, and the fp32 gate) and their float64 values."""
    hq, hkv, d = layer.hq, layer.hkv, layer.d
    n = (2 * hq + 2 * hkv) * d
    rng = np.random.default_rng(seed)
    in_norm = synth.f32_to_bf16_bits((0.1 * rng.standard_normal(hidden)).astype(np.float32))
    w_qkvg = synth.f32_to_bf16_bits((rng.standard_normal((n, hidden)) / np.sqrt(hidden)).astype(np.float32))
    w_o = synth.f32_to_bf16_bits((rng.standard_normal((hidden, hq * d)) / np.sqrt(hq * d)).astype(np.float32))
    W = {"in_norm": _f(in_norm), "w_qkvg": _f(w_qkvg), "w_o": _f(w_o)}
    dev = dict(in_norm=to_dev(in_norm), w_qkvg=to_dev(w_qkvg), w_o=to_dev(w_o))
    if spark:
        g = (0.5 * rng.standard_normal(hidden)).astype(np.float32)
        W["residual_gate"] = g.astype(np.float64)
        dev["residual_gate"] = torch.from_numpy(g).to(DEV)
    else:
        post = synth.f32_to_bf16_bits((0.1 * rng.standard_normal(hidden)).astype(np.float32))
        W["post_norm"] = _f(post)
        dev["post_norm"] = to_dev(post)
    return W, ma.BlockWeights(**dev)


CASES = [
    (Layer(hq=16, hkv=2, d=64, window=128, theta=10000.0, scale=SPARK_SCALE, out_norm=True, out_eps=1e-6), 768,
     True, 2, 200),
    (Layer(hq=16, hkv=2, d=64, window=0, theta=0.0, scale=SPARK_SCALE, out_norm=True, out_eps=1e-6), 1024, True, 1,
     300),
    (Layer(hq=32, hkv=2, d=128, window=0, theta=0.0, scale=GLIMMER_SCALE), 1024, False, 2, 150),
    (Layer(hq=32, hkv=2, d=128, window=64, theta=10000.0, scale=GLIMMER_SCALE), 640, False, 1, 130),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{'spark' if c[2] else 'glimmer'}-d{c[0].d}w{c[0].window}"
                                                      f"h{c[1]}")
def test_block_prefill_parity(case):
    layer, hidden, spark, B, T = case
    W, bw = make_block(layer, hidden, spark)
    xb = synth.normal_bf16_bits(3, 9, (B, T, hidden))
    y = ma.attention_block_prefill(ma.LayerParams.from_layer(layer), bw, to_dev(xb))
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    worst = 0.0
    for b in range(B):
        ref = OB.attention_block(_f(xb)[b], W, layer)
        worst = max(worst, max_err(y[b], ref))
    print(f"block {layer} hidden={hidden} B={B} T={T} max_abs_err={worst:.3e}", flush=True)
    assert worst <= BLOCK_TOL


def test_block_prefill_fullsize_spark_sampled():
    """Spark's width (8192, 128/16 heads of 64, a local layer) on 4096 tokens:
    sampled early rows against the oracle; every row finite, and with unit-RMS
    inputs the gated output's RMS stays within sqrt(2 * 1.001)."""
    layer = Layer(hq=128, hkv=16, d=64, window=2048, theta=10000.0, scale=SPARK_SCALE, out_norm=True, out_eps=1e-6)
    hidden, T = 8192, 4096
    W, bw = make_block(layer, hidden, True, seed=1)
    x = synth.normal_bf16_torch_tensor(4, 9, (1, T, hidden), DEV)
    y = ma.attention_block_prefill(ma.LayerParams.from_layer(layer), bw, x)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    rms = y.float().pow(2).mean(dim=-1).sqrt()
    assert float(rms.max()) <= np.sqrt(2 * 1.001) + 0.02
    rows = np.array([0, 1, 2, 63, 64, 127, 128, 200, 255])
    xh = x[0, :256].float().cpu().numpy().astype(np.float64)
    ref = OB.attention_block(xh, W, layer, rows=rows)
    err = max_err(y[0, rows].float().cpu().numpy(), ref)
    print(f"block full size spark: rows {rows.tolist()} max_abs_err={err:.3e}", flush=True)
    assert err <= BLOCK_TOL
