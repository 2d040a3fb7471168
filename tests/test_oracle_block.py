"""Pins of the block oracle (the attention half of a decoder block around
the layer): the pages' residual-gate table, four-channel example and figure
points, the RMSNorm epsilon floors, and an independent PyTorch formulation
of the whole block (rms_norm with a weight, linear, the layer's own library
pin formulation, sigmoid), with planted mistakes shown to fail it."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import block as OB
from synth.workloads import Layer, GLIMMER_SCALE, SPARK_SCALE

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def test_residual_gate_table():
    t = GOLD["residual_gate_table"]
    for row in t["rows"]:
        w = row["g"] / t["temperature"]
        beta = 1 / (1 + np.exp(-w))
        out_x = OB.residual_gate(1.0, 0.0, row["g"], t["temperature"], t["alpha_sq_floor"])   # alpha
        out_f = OB.residual_gate(0.0, 1.0, row["g"], t["temperature"], t["alpha_sq_floor"])   # beta
        digits = len(str(row["beta"]).split(".")[1])
        assert round(float(out_f), digits) == round(row["beta"], digits)
        assert round(float(out_x), len(str(row["alpha"]).split(".")[1])) == row["alpha"]
        assert round(float(out_x) ** 2 + float(out_f) ** 2, 4) == row["alpha2_plus_beta2"]
        assert round(float(np.degrees(np.arctan2(out_f, out_x))), 1) == row["theta_deg"]
        assert np.isclose(out_f, beta)
    # the clamp starts where alpha^2 = 1 - beta^2 reaches the floor
    g_on = t["temperature"] * np.log(t["clamp_onset_beta"] / (1 - t["clamp_onset_beta"]))
    assert round(g_on, 2) == t["clamp_onset_g"]


def test_residual_gate_four_channels_and_figure():
    e = GOLD["residual_gate_four_channels"]
    x, f = np.array(e["x"], float), np.array(e["f"], float)
    s = x + f
    assert np.array_equal(s, e["sum"]) and round(float(np.sqrt(np.mean(s * s))), 3) == e["sum_rms"]
    y = OB.residual_gate(x, f, np.full(4, e["g"]))
    assert np.allclose(np.round(y, 3), e["gated"]) and round(float(np.sqrt(np.mean(y * y))), 3) == e["gated_rms"]
    fig = GOLD["residual_gate_figure"]
    for pt in fig["points"]:
        g = 0.3 * np.log(pt["beta"] / (1 - pt["beta"]))
        a = float(OB.residual_gate(1.0, 0.0, g))
        assert round(a, 3) == pt["alpha"] and round(float(np.degrees(np.arcsin(pt["beta"]))), 1) == pt["deg"]
    assert round(float(OB.residual_gate(1.0, 0.0, 10.0)), 3) == fig["clamp_alpha_min"]


def test_rmsnorm_eps_floors():
    """Output RMS sqrt(ms / (ms + eps)) reaches 0.99 at the printed input RMS."""
    e = GOLD["rmsnorm_eps_floor"]
    for eps, key, nd in ((1e-5, "eps_1e-5_input_rms_for_0.99", 3), (1e-8, "eps_1e-8_input_rms_for_0.99", 4)):
        thr = np.sqrt(eps * 0.99 ** 2 / (1 - 0.99 ** 2))
        assert round(thr, nd) == e[key]
        out = float(np.sqrt(np.mean(OB.centered_rmsnorm(np.full(64, thr), 0.0, eps) ** 2)))
        assert abs(out - 0.99) < 1e-12


def torch_block(x, W, layer):
    import torch
    F = torch.nn.functional
    from test_oracle_pins import torch_reference
    tx = torch.from_numpy(x).double()
    hq, hkv, d = layer.hq, layer.hkv, layer.d
    h = F.rms_norm(tx, (x.shape[1],), weight=1 + torch.from_numpy(W["in_norm"]).double(), eps=1e-5)
    p = F.linear(h, torch.from_numpy(W["w_qkvg"]).double())
    T = x.shape[0]
    q = p[:, :hq * d].reshape(T, hq, d).numpy()
    k = p[:, hq * d:(hq + hkv) * d].reshape(T, hkv, d).numpy()
    v = p[:, (hq + hkv) * d:(hq + 2 * hkv) * d].reshape(T, hkv, d).numpy()
    g = p[:, (hq + 2 * hkv) * d:].reshape(T, hq, d).numpy()
    o = torch.from_numpy(torch_reference(q, k, v, g, layer, np.arange(T))).reshape(T, hq * d)
    a = F.linear(o, torch.from_numpy(W["w_o"]).double())
    if W.get("residual_gate") is not None:
        f = F.rms_norm(a, (x.shape[1],), eps=1e-8)
        beta = torch.sigmoid(torch.from_numpy(W["residual_gate"]).double() / 0.3)
        alpha = torch.sqrt(torch.clamp(1 - beta * beta, min=1e-3))
        return (alpha * tx + beta * f).numpy()
    return (tx + F.rms_norm(a, (x.shape[1],), weight=1 + torch.from_numpy(W["post_norm"]).double(),
                            eps=1e-8)).numpy()


def block_weights(rng, hidden, layer, spark):
    hq, hkv, d = layer.hq, layer.hkv, layer.d
    W = {"in_norm": 0.1 * rng.standard_normal(hidden),
         "w_qkvg": rng.standard_normal(((2 * hq + 2 * hkv) * d, hidden)) / np.sqrt(hidden),
         "w_o": rng.standard_normal((hidden, hq * d)) / np.sqrt(hq * d)}
    if spark:
        W["residual_gate"] = 0.5 * rng.standard_normal(hidden)
    else:
        W["post_norm"] = 0.1 * rng.standard_normal(hidden)
    return W


BLOCK_LAYERS = [(Layer(hq=8, hkv=2, d=16, window=7, theta=10000.0, scale=SPARK_SCALE, out_norm=True, out_eps=1e-6),
                 True, 48),
                (Layer(hq=4, hkv=1, d=32, window=0, theta=0.0, scale=GLIMMER_SCALE), False, 40)]


@pytest.mark.parametrize("layer,spark,hidden", BLOCK_LAYERS, ids=["spark-like", "glimmer-like"])
def test_block_matches_library_formulation(layer, spark, hidden):
    rng = np.random.default_rng(60)
    T = 21
    x = rng.standard_normal((T, hidden))
    W = block_weights(rng, hidden, layer, spark)
    y = OB.attention_block(x, W, layer)
    ref = torch_block(x, W, layer)
    assert np.allclose(y, ref, rtol=0, atol=1e-11)
    rows = np.array([0, 5, T - 1])
    assert np.allclose(OB.attention_block(x, W, layer, rows=rows), y[rows], rtol=0, atol=1e-13)


@pytest.mark.parametrize("mistake", ["gain_without_one", "gate_without_temperature", "post_norm_with_gain",
                                     "plain_add_on_spark"])
def test_planted_block_mistakes_fail_the_library_pin(monkeypatch, mistake):
    layer, spark, hidden = BLOCK_LAYERS[0]
    rng = np.random.default_rng(61)
    T = 12
    x = rng.standard_normal((T, hidden))
    W = block_weights(rng, hidden, layer, spark)
    ref = torch_block(x, W, layer)
    if mistake == "gain_without_one":
        monkeypatch.setattr(OB, "centered_rmsnorm", lambda x_, w, eps: OB.rms_normalize(x_, eps) * w)
    elif mistake == "gate_without_temperature":
        orig = OB.residual_gate
        monkeypatch.setattr(OB, "residual_gate", lambda x_, f, g, temperature=0.3, alpha_sq_floor=1e-3:
                            orig(x_, f, g, 1.0, alpha_sq_floor))
    elif mistake == "post_norm_with_gain":
        # Spark's post-attention norm is weightless; a stray gain fails the pin
        orig_rms = OB.rms_normalize
        monkeypatch.setattr(OB, "rms_normalize", lambda a, eps: orig_rms(a, eps) * (1.5 if eps == 1e-8 else 1.0))
    elif mistake == "plain_add_on_spark":
        monkeypatch.setattr(OB, "residual_gate", lambda x_, f, g, temperature=0.3, alpha_sq_floor=1e-3: x_ + f)
    y = OB.attention_block(x, W, layer)
    assert not np.allclose(y, ref, rtol=0, atol=1e-11)


@pytest.mark.parametrize("layer,spark,hidden", BLOCK_LAYERS, ids=["spark-like", "glimmer-like"])
def test_block_decode_equals_last_row_of_prefill_block(layer, spark, hidden):
    """A one-token decode block over a history holding the sequence's own earlier
    keys (normalized and rotated, unrounded) and values equals the last row of the
    prefill block on the whole sequence; a history one key short is rejected."""
    rng = np.random.default_rng(62)
    T = 19
    x = rng.standard_normal((T, hidden))
    W = block_weights(rng, hidden, layer, spark)
    _, k, v, _ = OB.input_projections(x, W, layer)
    kh = oracle.key_prologue(k, np.arange(T), layer)
    y_dec = OB.attention_block_decode(x[T - 1], W, layer, kh[:T - 1], v[:T - 1], 0, T)
    y_pre = OB.attention_block(x, W, layer)[T - 1]
    assert np.allclose(y_dec, y_pre, rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        OB.attention_block_decode(x[T - 1], W, layer, kh[:T - 2], v[:T - 2], 0, T)
