"""GPU parity of the attention half of a decoder block (input norm,
projections through hipBLASLt, the layer, o_proj, post-norm and residual)
against the fp64 block oracle, through the C ABI.

The bar is the layer's, TOL = 2e-2 max-abs, on the error beyond the block
output's own bf16 quantum.  The block returns the residual stream, whose
values reach 5-6 in magnitude; there one bf16 unit in the last place is
2^-5 = 0.031, so the correctly rounded oracle value itself sits up to 0.016
from the fp64 result.  Each output y is therefore held to
|y - ref| <= TOL + ulp_bf16(y) / 2, i.e. within TOL before its final
rounding (equivalently, max-abs 2e-2 on every output below magnitude 1,
where half an ulp is at most 2^-9).  On the device every intermediate
keeps at least fp16 precision except v and o (bf16, the operand type of the
layer's value product and of o_proj): h goes into the projection GEMM as a
bf16 hi/lo pair, the GEMMs accumulate and write fp32, q, k and the gate
reach the layer in fp16, and o_proj's output stays fp32.  An fp64 model of
exactly those roundings sits 0.6-1.2e-2 beyond half an ulp of the oracle on
these shapes; storing h, the projections and o_proj's output in bf16 put it
at 3.4-4.2e-2.
"""
import numpy as np
import pytest
import torch

import global_muse_rope_amd as ma
import synth
from oracle import block as OB
from synth.workloads import Layer, GLIMMER_SCALE, SPARK_SCALE
from gpu_helpers import TOL, to_dev, max_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def beyond_half_ulp(y, ref):
    """max over outputs of |y - ref| - ulp_bf16(y) / 2 (y holds bf16 values)."""
    y = np.asarray(y, dtype=np.float64)
    half_ulp = np.spacing(np.abs(y).astype(np.float32)).astype(np.float64) * 65536.0 / 2
    return float(np.max(np.abs(y - ref) - half_ulp))


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
    worst, plain = -1.0, 0.0
    for b in range(B):
        ref = OB.attention_block(_f(xb)[b], W, layer)
        worst = max(worst, beyond_half_ulp(y[b], ref))
        plain = max(plain, max_err(y[b], ref))
    print(f"block {layer} hidden={hidden} B={B} T={T} beyond half an ulp {worst:.3e} (max_abs_err {plain:.3e})",
          flush=True)
    assert worst <= TOL


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
    yr = y[0, rows].float().cpu().numpy()
    err = beyond_half_ulp(yr, ref)
    print(f"block full size spark: rows {rows.tolist()} beyond half an ulp {err:.3e} "
          f"(max_abs_err {max_err(yr, ref):.3e})", flush=True)
    assert err <= TOL


DEC_BLOCK_CASES = [
    # (kind, layer, hidden, spark, kv lengths, page_tokens)
    ("ring", Layer(hq=16, hkv=2, d=64, window=256, theta=10000.0, scale=SPARK_SCALE, out_norm=True, out_eps=1e-6),
     768, True, [1, 2, 255, 256, 1000], 0),
    ("paged", Layer(hq=16, hkv=2, d=64, window=0, theta=0.0, scale=SPARK_SCALE, out_norm=True, out_eps=1e-6),
     1024, True, [300, 77, 1, 33], 32),
    ("paged", Layer(hq=32, hkv=2, d=128, window=0, theta=0.0, scale=GLIMMER_SCALE), 1024, False, [500, 17, 2], 16),
]


@pytest.mark.parametrize("use_fp8", [False, True], ids=["bf16", "e4m3"])
@pytest.mark.parametrize("case", DEC_BLOCK_CASES, ids=lambda c: f"{c[0]}-hq{c[1].hq}d{c[1].d}w{c[1].window}")
def test_block_decode_parity(case, use_fp8):
    """One new token per sequence through the block over a cache of stored entries
    (bf16, or E4M3 codes with scales): every output against the block oracle's decode
    step over the stored (dequantized) history, and for bf16 the appended value rows."""
    from test_gpu_parity import make_cache, make_cache_fp8
    kind, layer, hidden, spark, lens, pt = case
    B = len(lens)
    lens = np.array(lens, dtype=np.int32)
    W, wb = make_block(layer, hidden, spark, seed=5)
    if use_fp8:
        cache, hk, hv, _, _ = make_cache_fp8(kind, layer, B, lens, page_tokens=pt or 32)
    else:
        cache, hk, hv = make_cache(kind, layer, B, lens, page_tokens=pt or 32)
    xb = synth.normal_bf16_bits(7, 9, (B, hidden))
    lp = ma.LayerParams.from_layer(layer)
    y = ma.attention_block_decode(lp, wb, to_dev(xb), torch.from_numpy(lens).to(DEV), int(lens.max()), cache)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    worst, plain = -1.0, 0.0
    for b in range(B):
        L = int(lens[b])
        ref = OB.attention_block_decode(_f(xb)[b], W, layer, hk[b, :L - 1].astype(np.float64),
                                        hv[b, :L - 1].astype(np.float64), 0, L)
        worst = max(worst, beyond_half_ulp(y[b], ref))
        plain = max(plain, max_err(y[b], ref))
    print(f"block decode {kind} fp8={use_fp8} {layer} hidden={hidden} beyond half an ulp {worst:.3e} "
          f"(max_abs_err {plain:.3e})", flush=True)
    assert worst <= TOL
    if use_fp8:
        return
    # the new value row landed in the cache (the bf16 rounding of the fp32 projection of the normed
    # input, so compare with the oracle's projection within half a bf16 ulp plus the GEMM's error)
    _, _, v_new, _ = OB.input_projections(_f(xb), W, layer)
    for b in range(B):
        p = int(lens[b]) - 1
        if kind == "ring":
            vst = cache.v[b, :, :, p % layer.window].float().cpu().numpy()
        else:
            pg = int(cache.block_table[b, p // pt])
            vst = cache.v[pg, :, :, p % pt].float().cpu().numpy()
        assert np.allclose(vst, v_new[b], rtol=2 ** -8, atol=1e-3)


def test_block_decode_fullsize_ring():
    """The Spark local decode workload (16 sequences, a 2048-entry ring, lengths in
    [131072, 1048576]) through a block of hidden width 8192: every sequence against
    the block oracle over its stored window."""
    from synth import device as sd
    from synth import workloads as wl
    from synth.device import block_device_setup
    cfg = wl.SPARK_DECODE_LOCAL
    L = cfg.layer
    bcfg = wl.SPARK_BLOCK_LOCAL
    assert bcfg.layer == L
    print(f"block decode full size {cfg.name}", flush=True)
    s = sd.decode_device_setup(cfg)
    cache = ma.KvCache.ring(s["kc"], s["vc"])
    w = block_device_setup(bcfg)
    wb = ma.BlockWeights(in_norm=w["in_norm"], w_qkvg=w["w_qkvg"], w_o=w["w_o"], residual_gate=w["residual_gate"],
                         post_norm=w["post_norm"])
    B = cfg.batch
    x = synth.normal_bf16_torch_tensor(cfg.seed, 9, (B, bcfg.hidden), DEV)
    lp = ma.LayerParams.from_layer(L)
    y = ma.attention_block_decode(lp, wb, x, s["kv_len"], s["max_len"], cache)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()

    def host(t):
        return t.double().cpu().numpy() if t is not None else None

    Wt = {"in_norm": host(w["in_norm"]), "w_qkvg": host(w["w_qkvg"]), "w_o": host(w["w_o"]),
          "post_norm": host(w["post_norm"]), "residual_gate": host(w["residual_gate"])}
    xh = x.double().cpu().numpy()
    worst, plain = -1.0, 0.0
    for b in range(B):
        Lb = int(s["lengths"][b])
        p = Lb - 1
        lo = max(0, p - L.window + 1)
        kh = np.stack([sd.cache_values_host(cfg.seed, b, h, L.hkv, "k", lo, p, L.d) for h in range(L.hkv)], axis=1)
        vh = np.stack([sd.cache_values_host(cfg.seed, b, h, L.hkv, "v", lo, p, L.d) for h in range(L.hkv)], axis=1)
        ref = OB.attention_block_decode(xh[b], Wt, L, kh, vh, lo, Lb)
        worst = max(worst, beyond_half_ulp(y[b], ref))
        plain = max(plain, max_err(y[b], ref))
    print(f"{cfg.name} through the block: {B} sequences, beyond half an ulp {worst:.3e} (max_abs_err {plain:.3e})",
          flush=True)
    assert worst <= TOL
