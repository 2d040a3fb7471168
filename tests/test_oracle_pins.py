"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (tests/golden/page_values.json, each with its citation), closed
forms, invariants, an independent library formulation (PyTorch's rms_norm,
complex multiplication and scaled_dot_product_attention in float64), and a
50-digit mpmath evaluation on tiny inputs.  test_planted_mistakes shows that
plausible slips in the oracle fail these pins.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import Layer, GLIMMER_SCALE, SPARK_SCALE

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def rounded_eq(x, value, digits):
    return round(float(x), digits) == round(float(value), digits)


def spark_layer(**kw):
    base = dict(hq=8, hkv=1, d=64, window=0, theta=0.0, scale=SPARK_SCALE)
    base.update(kw)
    return Layer(**base)


def glimmer_layer(**kw):
    base = dict(hq=16, hkv=1, d=128, window=0, theta=0.0, scale=GLIMMER_SCALE)
    base.update(kw)
    return Layer(**base)


def logit(q, k, layer, pos=(0, 0)):
    qh = oracle.query_prologue(np.asarray(q)[None, None], [pos[0]], layer)
    kh = oracle.key_prologue(np.asarray(k)[None, None], [pos[1]], layer)
    return float(oracle.logits_for_row(qh[0], kh, 1)[0, 0])


# --------------------------------------------------------------------------
# Layer schedule and visibility (integer logic)
# --------------------------------------------------------------------------

def test_layer_types_match_pages():
    lt = GOLD["layer_types"]
    assert oracle.global_layers(lt["glimmer"]["n_layers"]) == lt["glimmer"]["global"]
    assert oracle.global_layers(lt["spark"]["n_layers"]) == lt["spark"]["global"]
    forward = [i for i in range(62) if (i + 1) % 4 == 0]
    assert len(forward) == lt["spark_forward_rule_count"]
    assert forward != lt["spark"]["global"]


def test_window_includes_self():
    w = GOLD["window_includes_self"]["window"]
    i = 10 * w
    lo, hi = oracle.visible_range(i, w)
    assert hi == i and hi - lo + 1 == GOLD["window_includes_self"]["visible_with_self"]
    assert oracle.visible_range(5, w) == (0, 5)
    assert oracle.visible_range(5, 0) == (0, 5)
    assert oracle.visible_range(10 * w, 0) == (0, 10 * w)


def test_bidirectional_range_brute_force():
    """The drafter's two-sided window (deep dive, section 8.2, step 4: no causal
    mask inside the window) against the set {j <= last : |p - j| < W}, or every
    key up to last on a window-0 layer, enumerated directly; a position well
    inside sees 2W - 1 keys, the self key counted once."""
    for w in (0, 1, 2, 5, 64):
        for last in (0, 3, 70, 200):
            for p in range(0, last + 1):
                want = [j for j in range(0, last + 1) if w == 0 or abs(p - j) < w]
                lo, hi = oracle.bidirectional_range(p, w, last)
                assert list(range(lo, hi + 1)) == want, (w, last, p)
    lo, hi = oracle.bidirectional_range(5000, 2048, 10 ** 6)
    assert hi - lo + 1 == 2 * 2048 - 1


def test_visible_counts_closed_form():
    from global_muse_rope_amd import accounting
    for n, w in [(1, 1), (7, 1), (64, 5), (100, 100), (100, 200), (1024, 256), (1024, 0), (333, 64)]:
        m = oracle.visible_mask(n, w)
        counts = m.sum(axis=1)
        expect = np.minimum(np.arange(n) + 1, w if w else n + 1)
        assert np.array_equal(counts, expect)
        assert int(m.sum()) == accounting.visible_pairs(n, w)
    assert accounting.visible_pairs(1024, 256) == 229504
    assert accounting.visible_pairs(1024, 0) == 524800


def test_stacked_receptive_field():
    """Three stacked causal windows reach 1 + 3(W - 1) positions."""
    g = GOLD["stacked_receptive_field"]
    for w, expect in [(g["window"], g["value"]), (256, 1 + 3 * 255)]:
        n = 3 * (w - 1) + 40
        m = oracle.visible_mask(n, w).astype(np.int32)
        row = np.zeros(n, dtype=np.int32)
        row[n - 1] = 1
        for _ in range(3):
            # keys reachable in one more layer: union of the windows of the current set
            row = ((row @ m) > 0).astype(np.int32)
        assert int(row.sum()) == expect
    r = GOLD["mistral_reach"]
    assert 46 * 2047 == r["spark"] and 39 * 2047 == r["glimmer"]


# --------------------------------------------------------------------------
# QK-norm, multiplier and the logit bound
# --------------------------------------------------------------------------

def test_scale_constants():
    num = GOLD["logit_numerator"]["value"]
    assert abs(GOLD["spark_scale"]["value"] * math.sqrt(64) - num) < 1e-9
    assert abs(GOLD["glimmer_scale"]["value"] * math.sqrt(128) - num) < 1e-9


def test_logit_worked_examples():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(64)
    x = x / np.sqrt(np.mean(x * x))           # unit RMS, so the eps effect is 1/(1+1e-5)
    sp = spark_layer()
    l_al = logit(x, x, sp)
    assert rounded_eq(l_al, GOLD["logit_aligned_spark"]["value"], 2)
    # a key at 60 degrees: x cos60 + y sin60 with y orthogonal to x, unit RMS
    y = rng.standard_normal(64)
    y -= (y @ x) / (x @ x) * x
    y = y / np.sqrt(np.mean(y * y))
    k60 = 0.5 * x + math.sqrt(3) / 2 * y
    assert rounded_eq(logit(x, k60, sp), GOLD["logit_60deg_spark"]["value"], 2)
    z = rng.standard_normal(128)
    assert rounded_eq(logit(z, z, glimmer_layer()), GOLD["logit_aligned_glimmer"]["value"], 2)


@pytest.mark.parametrize("case", GOLD["bound_with_eps"]["cases"])
def test_bound_with_eps(case):
    """Aligned q and k with mean square m reach 43.784 m / (m + 1e-5)."""
    m = case["m"]
    for layer, d in [(spark_layer(), 64), (glimmer_layer(), 128)]:
        x = np.full(d, math.sqrt(m))
        assert rounded_eq(logit(x, x, layer), case["value"], case["digits"])


def test_logit_bound_any_input():
    rng = np.random.default_rng(2)
    bound = GOLD["logit_numerator"]["value"]
    for layer in [spark_layer(window=16, theta=10000.0), glimmer_layer()]:
        d = layer.d
        worst = 0.0
        for trial in range(200):
            scale = 10.0 ** rng.uniform(-3, 3)
            q = rng.standard_normal((1, 1, d)) * scale
            k = rng.standard_normal((64, 1, d)) * 10.0 ** rng.uniform(-3, 3, size=(64, 1, 1))
            if trial % 3 == 0:
                k[:, 0, :] = q[0, 0] * rng.uniform(0.1, 10)       # aligned keys
            pos = np.arange(64)
            qh = oracle.query_prologue(q, [63], layer)
            kh = oracle.key_prologue(k, pos, layer)
            lg = oracle.logits_for_row(qh[0], kh, 1)
            worst = max(worst, float(np.max(np.abs(lg))))
        assert worst <= bound * (1 + 1e-12)
        assert worst > 0.9 * bound


def test_typical_spread_on_synthetic_inputs():
    for layer, target in [(spark_layer(), GOLD["typical_spread"]["spark"]),
                          (glimmer_layer(), GOLD["typical_spread"]["glimmer"])]:
        d = layer.d
        q = synth.bf16_bits_to_f64(synth.normal_bf16_bits(0, 1, (256, 1, d)))
        k = synth.bf16_bits_to_f64(synth.normal_bf16_bits(0, 2, (256, 1, d)))
        qh, kh = oracle.qk_prologue(q, k, np.arange(256), layer)
        lg = (qh[:, 0, :] @ kh[:, 0, :].T) / math.sqrt(d)
        assert abs(np.std(lg) / target - 1) < 0.05


def test_norm_is_unit_rms_and_v_untouched():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 3, 64)) * 7
    y = oracle.rms_normalize(x, 1e-5)
    ms = np.mean(x * x, axis=-1)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), np.sqrt(ms / (ms + 1e-5)), rtol=1e-14)


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------

def test_rope_frequency_facts():
    f = GOLD["rope_facts_theta_500000_window_2048"]
    theta = GOLD["rope_theta_pages"]["value"]
    for name, d in [("spark", 64), ("glimmer", 128)]:
        inv = oracle.rope_inv_freq(d, theta)
        assert len(inv) == f[f"{name}_pairs"]
        turned = inv * 2048
        assert int(np.sum(turned >= 2 * math.pi)) == f["full_turn"][name]
        assert int(np.sum(turned < math.pi / 2)) == f["under_90_deg"][name]
        assert int(np.sum(turned < math.radians(10))) == f["under_10_deg"][name]
    inv64 = oracle.rope_inv_freq(64, theta)
    assert rounded_eq(math.degrees(inv64[-1] * 2048), f["slowest_spark_deg_per_window"]["value"], 2)
    assert rounded_eq(2 * math.pi / inv64[0], f["fastest_period_tokens"]["value"], 1)


def test_rope_equals_complex_rotation():
    """RoPE as the complex product z_j * exp(i p w_j), z_j = x_j + i x_{j+D/2}."""
    rng = np.random.default_rng(4)
    for d, theta in [(64, 10000.0), (128, 500000.0), (8, 3.0)]:
        x = rng.standard_normal((9, 2, d))
        pos = rng.integers(0, 1 << 20, size=9)
        got = oracle.rope_rotate(x, pos, theta)
        h = d // 2
        w = theta ** (-np.arange(h) * 2.0 / d)
        z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * (pos[:, None, None] * w[None, None, :]))
        ref = np.concatenate([z.real, z.imag], axis=-1)
        assert np.allclose(got, ref, rtol=0, atol=1e-9)


def test_rope_pairs_j_with_j_plus_half():
    d = 16
    for j in range(d):
        e = np.zeros((1, 1, d))
        e[0, 0, j] = 1.0
        r = oracle.rope_rotate(e, [3], 10.0)[0, 0]
        nz = set(np.flatnonzero(np.abs(r) > 1e-15).tolist())
        assert nz <= {j, (j + d // 2) % d}
        assert np.isclose(np.linalg.norm(r), 1.0)


def test_rope_relative_position_and_commutes_with_norm():
    rng = np.random.default_rng(5)
    layer = spark_layer(window=64, theta=10000.0)
    q = rng.standard_normal((6, 1, 64))
    k = rng.standard_normal((6, 1, 64))
    pos = np.array([0, 5, 9, 100, 1000, 4095])
    for shift in [1, 77, 123456]:
        qa, ka = oracle.qk_prologue(q, k, pos, layer)
        qb, kb = oracle.qk_prologue(q, k, pos + shift, layer)
        la = qa[:, 0] @ ka[:, 0].T
        lb = qb[:, 0] @ kb[:, 0].T
        assert np.allclose(la, lb, rtol=0, atol=1e-9)
    # rotation preserves the RMS, so norm(rope(x)) == rope(norm(x))
    a = oracle.rms_normalize(oracle.rope_rotate(q, pos, 10000.0), 1e-5)
    b = oracle.rope_rotate(oracle.rms_normalize(q, 1e-5), pos, 10000.0)
    assert np.allclose(a, b, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Softmax, GQA, window, epilogue
# --------------------------------------------------------------------------

def _rand_layer_inputs(rng, t, layer):
    q = rng.standard_normal((t, layer.hq, layer.d))
    k = rng.standard_normal((t, layer.hkv, layer.d))
    v = rng.standard_normal((t, layer.hkv, layer.d))
    g = rng.standard_normal((t, layer.hq, layer.d))
    return q, k, v, g


def test_softmax_special_cases():
    rng = np.random.default_rng(6)
    layer = Layer(hq=4, hkv=2, d=16, window=3, theta=100.0, scale=2.0)
    q, k, v, g = _rand_layer_inputs(rng, 20, layer)
    qh, kh = oracle.qk_prologue(q, k, np.arange(20), layer)
    o = oracle.attend_rows(qh, np.arange(20), kh, v, layer)
    # row 0 sees only itself: o = v_0 exactly
    for h in range(4):
        assert np.array_equal(o[0, h], v[0, h // 2])
    # weights of every row sum to one
    for i in range(20):
        lo, hi = oracle.visible_range(i, 3)
        w = oracle.softmax(oracle.logits_for_row(qh[i], kh[lo:hi + 1], 2))
        assert np.allclose(w.sum(axis=1), 1.0, atol=1e-14)
    # identical keys: o = mean of the visible values
    k_same = np.repeat(k[:1], 20, axis=0)
    kh2 = oracle.key_prologue(k_same, np.zeros(20), layer)
    o2 = oracle.attend_rows(qh, np.arange(20), kh2, v, layer)
    for i in range(20):
        lo, hi = oracle.visible_range(i, 3)
        for h in range(4):
            assert np.allclose(o2[i, h], v[lo:hi + 1, h // 2].mean(axis=0), atol=1e-14)
    # constant values: o = that value
    v_c = np.broadcast_to(np.arange(16.0), v.shape)
    o3 = oracle.attend_rows(qh, np.arange(20), kh, v_c, layer)
    assert np.allclose(o3, np.arange(16.0), atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(7)
    gqa = Layer(hq=8, hkv=2, d=16, window=5, theta=1000.0, scale=3.0, out_norm=True)
    mha = Layer(hq=8, hkv=8, d=16, window=5, theta=1000.0, scale=3.0, out_norm=True)
    q, k, v, g = _rand_layer_inputs(rng, 24, gqa)
    y1 = oracle.prefill(q, k, v, g, gqa)
    y2 = oracle.prefill(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), g, mha)
    assert np.allclose(y1, y2, rtol=0, atol=1e-14)


def test_window_at_least_sequence_equals_global():
    rng = np.random.default_rng(8)
    loc = Layer(hq=4, hkv=1, d=32, window=40, theta=10000.0, scale=3.87)
    glo = Layer(hq=4, hkv=1, d=32, window=0, theta=10000.0, scale=3.87)
    q, k, v, g = _rand_layer_inputs(rng, 40, loc)
    assert np.array_equal(oracle.prefill(q, k, v, g, loc), oracle.prefill(q, k, v, g, glo))
    loc39 = Layer(hq=4, hkv=1, d=32, window=39, theta=10000.0, scale=3.87)
    assert not np.allclose(oracle.prefill(q, k, v, g, loc39), oracle.prefill(q, k, v, g, glo))


def test_output_norm_per_head_and_gate_examples():
    ge = GOLD["gate_examples"]
    plain = Layer(hq=1, hkv=1, d=1, window=0, theta=0.0, scale=1.0)
    for c in ge["cases"]:
        y = oracle.output_epilogue(np.array([[ge["o"]]]), np.array([[c["g"]]]), plain)
        assert rounded_eq(oracle.sigmoid(c["g"]), c["sigmoid"], 3)
        assert rounded_eq(y[0, 0], c["y"], 3 if c["y"] < 0.1 else 2)
    ch = ge["channel"]
    assert ch["head"] * ch["head_dim"] + ch["dim"] == ch["index"]
    rng = np.random.default_rng(9)
    layer = Layer(hq=4, hkv=1, d=64, window=0, theta=0.0, scale=1.0, out_norm=True, out_eps=1e-6)
    o = rng.standard_normal((3, 4, 64)) * np.array([0.1, 1.0, 3.0, 0.01])[None, :, None]
    y = oracle.output_epilogue(o, np.zeros_like(o), layer)
    ms = np.mean(o * o, axis=-1)
    # per head RMS sqrt(ms/(ms+eps)), then halved by the zero gate logits
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 0.5 * np.sqrt(ms / (ms + 1e-6)), rtol=1e-13)
    # a single norm over the whole Hq*D vector is a different function
    whole = o / np.sqrt(np.mean(o.reshape(3, -1) ** 2, axis=-1) + 1e-6)[:, None, None] * 0.5
    assert not np.allclose(y, whole, atol=1e-3)
    # gate logit 0 halves the output (no o_norm)
    y0 = oracle.output_epilogue(o, np.zeros_like(o), Layer(hq=4, hkv=1, d=64, window=0, theta=0.0, scale=1.0))
    assert np.array_equal(y0, o * 0.5)


# --------------------------------------------------------------------------
# Independent library formulation (PyTorch float64) and 50-digit brute force
# --------------------------------------------------------------------------

def torch_reference(q, k, v, g, layer, positions):
    """The layer from PyTorch library routines: rms_norm, complex rotation,
    scaled_dot_product_attention with a boolean mask and enable_gqa."""
    import torch
    import torch.nn.functional as F
    tq = torch.from_numpy(q).double()
    tk = torch.from_numpy(k).double()
    tv = torch.from_numpy(v).double()
    tg = torch.from_numpy(g).double()
    d = q.shape[-1]
    qh = F.rms_norm(tq, (d,), eps=layer.qk_eps) * layer.scale
    kh = F.rms_norm(tk, (d,), eps=layer.qk_eps)
    if layer.theta:
        h = d // 2
        freqs = torch.tensor(layer.theta, dtype=torch.float64) ** (-torch.arange(h, dtype=torch.float64) * 2 / d)
        ang = torch.tensor(positions, dtype=torch.float64)[:, None] * freqs[None, :]
        rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]

        def apply(x):
            z = torch.complex(x[..., :h], x[..., h:]) * rot
            return torch.cat([z.real, z.imag], dim=-1)
        qh, kh = apply(qh), apply(kh)
    t = q.shape[0]
    i = torch.arange(t)[:, None]
    j = torch.arange(t)[None, :]
    mask = j <= i
    if layer.window:
        mask &= j > i - layer.window
    o = F.scaled_dot_product_attention(qh.transpose(0, 1)[None], kh.transpose(0, 1)[None],
                                       tv.transpose(0, 1)[None], attn_mask=mask, enable_gqa=True)
    o = o[0].transpose(0, 1)
    if layer.out_norm:
        o = F.rms_norm(o, (d,), eps=layer.out_eps)
    return (o * torch.sigmoid(tg)).numpy()


LIB_CASES = [
    Layer(hq=8, hkv=2, d=16, window=7, theta=10000.0, scale=SPARK_SCALE, out_norm=True, out_eps=1e-6),
    Layer(hq=8, hkv=2, d=16, window=0, theta=0.0, scale=SPARK_SCALE, out_norm=True, out_eps=1e-6),
    Layer(hq=6, hkv=3, d=32, window=5, theta=500000.0, scale=GLIMMER_SCALE),
    Layer(hq=4, hkv=1, d=8, window=0, theta=0.0, scale=GLIMMER_SCALE),
]


@pytest.mark.parametrize("layer", LIB_CASES, ids=lambda l: f"hq{l.hq}kv{l.hkv}d{l.d}w{l.window}")
def test_oracle_matches_torch_library_formulation(layer):
    rng = np.random.default_rng(10)
    t = 37
    q, k, v, g = _rand_layer_inputs(rng, t, layer)
    pos = np.arange(t) + 1000
    y = oracle.prefill(q, k, v, g, layer, positions=pos)
    ref = torch_reference(q, k, v, g, layer, pos)
    assert np.allclose(y, ref, rtol=0, atol=1e-12)


def test_oracle_rows_subset_matches_full():
    rng = np.random.default_rng(11)
    layer = LIB_CASES[0]
    q, k, v, g = _rand_layer_inputs(rng, 30, layer)
    full = oracle.prefill(q, k, v, g, layer)
    rows = np.array([0, 6, 7, 29])
    part = oracle.prefill(q[rows], k, v, g[rows], layer, rows=rows)
    assert np.array_equal(part, full[rows])


def test_mpmath_brute_force_tiny():
    mpmath = pytest.importorskip("mpmath")
    mp = mpmath.mp
    mp.dps = 50
    rng = np.random.default_rng(12)
    layer = Layer(hq=2, hkv=1, d=8, window=4, theta=10000.0, scale=SPARK_SCALE, out_norm=True, out_eps=1e-6)
    t = 9
    q, k, v, g = _rand_layer_inputs(rng, t, layer)
    y = oracle.prefill(q, k, v, g, layer)
    d, h = 8, 4

    def norm(x):
        ms = mp.fsum([mp.mpf(a) ** 2 for a in x]) / d
        return [mp.mpf(a) / mp.sqrt(ms + mp.mpf("1e-5")) for a in x]

    def rot(x, p):
        out = list(x)
        for j in range(h):
            a = p * mp.power(mp.mpf(10000), -mp.mpf(2 * j) / d)
            out[j] = x[j] * mp.cos(a) - x[j + h] * mp.sin(a)
            out[j + h] = x[j + h] * mp.cos(a) + x[j] * mp.sin(a)
        return out

    s = mp.mpf("5.4730064863875")
    keys = [rot(norm(k[j, 0]), j) for j in range(t)]
    for i in [0, 3, 8]:
        for hh in range(2):
            qq = rot([s * a for a in norm(q[i, hh])], i)
            vis = list(range(max(0, i - 3), i + 1))
            lg = [mp.fsum([qq[c] * keys[j][c] for c in range(d)]) / mp.sqrt(d) for j in vis]
            m = max(lg)
            e = [mp.exp(x - m) for x in lg]
            z = mp.fsum(e)
            o = [mp.fsum([e[n] * mp.mpf(v[j, 0, c]) for n, j in enumerate(vis)]) / z for c in range(d)]
            ms = mp.fsum([a * a for a in o]) / d
            o = [a / mp.sqrt(ms + mp.mpf("1e-6")) for a in o]
            ref = [o[c] / (1 + mp.exp(-mp.mpf(g[i, hh, c]))) for c in range(d)]
            assert max(abs(float(ref[c]) - y[i, hh, c]) for c in range(d)) < 1e-13


def test_decode_equals_last_prefill_row():
    rng = np.random.default_rng(13)
    for layer in [Layer(hq=8, hkv=2, d=16, window=6, theta=10000.0, scale=SPARK_SCALE, out_norm=True),
                  Layer(hq=8, hkv=2, d=16, window=0, theta=0.0, scale=GLIMMER_SCALE)]:
        t = 21
        q, k, v, g = _rand_layer_inputs(rng, t, layer)
        y = oracle.prefill(q, k, v, g, layer)
        _, kh = oracle.qk_prologue(q, k, np.arange(t), layer)
        yd = oracle.decode_one(q[-1], k[-1], v[-1], g[-1], kh[:t - 1], v[:t - 1], 0, t, layer)
        assert np.allclose(yd, y[-1], rtol=0, atol=1e-13)
        if layer.window:
            start = t - layer.window
            yd2 = oracle.decode_one(q[-1], k[-1], v[-1], g[-1], kh[start:t - 1], v[start:t - 1], start, t, layer)
            assert np.allclose(yd2, y[-1], rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# The pins catch plausible mistakes planted in the oracle (CPU only)
# --------------------------------------------------------------------------

def _adjacent_rope(x, positions, theta):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.asarray(positions, dtype=np.float64)[:, None] * oracle.rope_inv_freq(d, theta)[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    out = x.copy()
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 1::2] * c + x[..., 0::2] * s
    return out


def _sign_flip_rope(x, positions, theta):
    return oracle.attention.__dict__["_orig_rope"](x, -np.asarray(positions), theta)


def _interleaved_gqa_attend(qh_rows, row_index, kh, v, layer):
    """attend_rows with query head h mapped to KV head h mod Hkv (a plausible
    mix-up of the contiguous grouping)."""
    kh = np.asarray(kh, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(np.shape(qh_rows), dtype=np.float64)
    for r, i in enumerate(row_index):
        lo, hi = oracle.visible_range(int(i), layer.window)
        for h in range(layer.hq):
            kv = h % layer.hkv
            lg = kh[lo:hi + 1, kv, :] @ qh_rows[r, h] / np.sqrt(layer.d)
            w = oracle.softmax(lg)
            out[r, h] = w @ v[lo:hi + 1, kv, :]
    return out


@pytest.mark.parametrize("mistake", ["adjacent_pairs", "rope_sign", "eps_outside", "window_off_by_one",
                                     "whole_vector_onorm", "no_query_scale", "interleaved_gqa"])
def test_planted_mistakes_fail_the_library_pin(monkeypatch, mistake):
    import oracle.attention as A
    layer = LIB_CASES[0]
    if mistake == "adjacent_pairs":
        monkeypatch.setattr(A, "rope_rotate", _adjacent_rope)
    elif mistake == "rope_sign":
        A.__dict__["_orig_rope"] = A.rope_rotate
        monkeypatch.setattr(A, "rope_rotate", _sign_flip_rope)
    elif mistake == "eps_outside":
        monkeypatch.setattr(A, "rms_normalize",
                            lambda x, eps: np.asarray(x, float) / (np.sqrt(np.mean(np.asarray(x, float) ** 2, -1, keepdims=True)) + eps))
    elif mistake == "window_off_by_one":
        monkeypatch.setattr(A, "visible_range", lambda i, w: (0 if w == 0 else max(0, i - w), i))
    elif mistake == "whole_vector_onorm":
        def whole(o, gate, lyr):
            o = np.asarray(o, float)
            if lyr.out_norm:
                flat = o.reshape(o.shape[0], -1)
                o = o / np.sqrt(np.mean(flat * flat, -1) + lyr.out_eps)[:, None, None]
            return o * A.sigmoid(gate)
        monkeypatch.setattr(A, "output_epilogue", whole)
    elif mistake == "interleaved_gqa":
        monkeypatch.setattr(A, "attend_rows", _interleaved_gqa_attend)
    elif mistake == "no_query_scale":
        from dataclasses import replace
        orig = A.query_prologue
        monkeypatch.setattr(A, "query_prologue", lambda q, p, l, *rest: orig(q, p, replace(l, scale=1.0), *rest))
    rng = np.random.default_rng(10)
    q, k, v, g = _rand_layer_inputs(rng, 37, layer)
    pos = np.arange(37) + 1000
    y = A.prefill(q, k, v, g, layer, positions=pos)
    ref = torch_reference(q, k, v, g, layer, pos)
    assert not np.allclose(y, ref, rtol=0, atol=1e-6)


# --------------------------------------------------------------------------
# Chunked prefill: a chunk over a cached history is the tail of the whole
# sequence's prefill
# --------------------------------------------------------------------------

CHUNK_LAYERS = [Layer(hq=8, hkv=2, d=16, window=6, theta=10000.0, scale=SPARK_SCALE, out_norm=True, out_eps=1e-6),
                Layer(hq=8, hkv=2, d=16, window=0, theta=0.0, scale=GLIMMER_SCALE),
                Layer(hq=6, hkv=3, d=32, window=5, theta=500000.0, scale=GLIMMER_SCALE)]


@pytest.mark.parametrize("layer", CHUNK_LAYERS, ids=lambda l: f"hq{l.hq}kv{l.hkv}d{l.d}w{l.window}")
@pytest.mark.parametrize("start", [0, 1, 5, 6, 13])
def test_chunk_is_tail_of_whole_prefill(layer, start):
    rng = np.random.default_rng(20 + start)
    n = 23
    q, k, v, g = _rand_layer_inputs(rng, n, layer)
    full = oracle.prefill(q, k, v, g, layer)
    _, kh = oracle.qk_prologue(q, k, np.arange(n), layer)
    # history from position 0, and (local layers) only the window's part
    hist_starts = [0] + ([max(0, start - layer.window + 1)] if layer.window else [])
    for hs in hist_starts:
        y = oracle.prefill_chunk(q[start:], k[start:], v[start:], g[start:], kh[hs:start], v[hs:start], hs, start,
                                 layer)
        assert np.allclose(y, full[start:], rtol=0, atol=1e-13)
    rows = np.array([0, n - start - 1])
    yr = oracle.prefill_chunk(q[start:][rows], k[start:], v[start:], g[start:][rows], kh[:start], v[:start], 0,
                              start, layer, rows=rows)
    assert np.array_equal(yr, oracle.prefill_chunk(q[start:], k[start:], v[start:], g[start:], kh[:start],
                                                   v[:start], 0, start, layer)[rows])


def test_chunk_rejects_short_history():
    layer = CHUNK_LAYERS[0]
    rng = np.random.default_rng(30)
    q, k, v, g = _rand_layer_inputs(rng, 12, layer)
    _, kh = oracle.qk_prologue(q, k, np.arange(12), layer)
    with pytest.raises(ValueError):
        oracle.prefill_chunk(q[8:], k[8:], v[8:], g[8:], kh[4:8], v[4:8], 4, 8, layer)   # needs position 3


@pytest.mark.parametrize("mistake", ["positions_from_zero", "history_renormalized", "window_from_chunk_start"])
def test_planted_chunk_mistakes_fail_the_tail_pin(monkeypatch, mistake):
    import oracle.attention as A
    layer = CHUNK_LAYERS[0]
    rng = np.random.default_rng(31)
    n, start = 20, 9
    q, k, v, g = _rand_layer_inputs(rng, n, layer)
    full = oracle.prefill(q, k, v, g, layer)
    _, kh = oracle.qk_prologue(q, k, np.arange(n), layer)
    kh_hist = kh[:start]
    if mistake == "positions_from_zero":
        orig = A.key_prologue
        monkeypatch.setattr(A, "key_prologue", lambda x, pos, lyr: orig(x, np.asarray(pos) - start, lyr))
    elif mistake == "history_renormalized":
        kh_hist = A.rms_normalize(kh_hist, layer.qk_eps)
    elif mistake == "window_from_chunk_start":
        orig_vr = A.visible_range
        monkeypatch.setattr(A, "visible_range", lambda i, w: (max(orig_vr(i, w)[0], start), i))
    y = A.prefill_chunk(q[start:], k[start:], v[start:], g[start:], kh_hist, v[:start], 0, start, layer)
    assert not np.allclose(y, full[start:], rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# Non-causal block attention (block-diffusion drafter)
# --------------------------------------------------------------------------

def torch_block_reference(q, k, v, g, k_hist, v_hist, start, layer):
    """Independent formulation: PyTorch rms_norm, complex RoPE and SDPA with an
    explicit |i - j| < W mask over the concatenated [history; block] keys."""
    import torch
    F = torch.nn.functional
    d = q.shape[-1]
    T = q.shape[0]
    hs = start - k_hist.shape[0]
    pos_q = torch.arange(start, start + T, dtype=torch.float64)
    qh = F.rms_norm(torch.from_numpy(q).double(), (d,), eps=layer.qk_eps) * layer.scale
    kh = F.rms_norm(torch.from_numpy(k).double(), (d,), eps=layer.qk_eps)
    if layer.theta:
        h = d // 2
        freqs = torch.tensor(layer.theta, dtype=torch.float64) ** (-torch.arange(h, dtype=torch.float64) * 2 / d)
        rot = torch.polar(torch.ones(T, h, dtype=torch.float64), pos_q[:, None] * freqs[None, :])[:, None, :]

        def apply(x):
            z = torch.complex(x[..., :h], x[..., h:]) * rot
            return torch.cat([z.real, z.imag], dim=-1)
        qh, kh = apply(qh), apply(kh)
    keys = torch.cat([torch.from_numpy(k_hist).double(), kh])
    vals = torch.cat([torch.from_numpy(v_hist).double(), torch.from_numpy(v).double()])
    i = pos_q[:, None]
    j = torch.arange(hs, start + T, dtype=torch.float64)[None, :]
    mask = torch.ones(T, keys.shape[0], dtype=torch.bool)
    if layer.window:
        mask = (i - j).abs() < layer.window
    o = F.scaled_dot_product_attention(qh.transpose(0, 1)[None], keys.transpose(0, 1)[None],
                                       vals.transpose(0, 1)[None], attn_mask=mask, enable_gqa=True)[0].transpose(0, 1)
    if layer.out_norm:
        o = F.rms_norm(o, (d,), eps=layer.out_eps)
    return (o * torch.sigmoid(torch.from_numpy(g).double())).numpy()


@pytest.mark.parametrize("layer", CHUNK_LAYERS, ids=lambda l: f"hq{l.hq}kv{l.hkv}d{l.d}w{l.window}")
@pytest.mark.parametrize("start,T", [(0, 7), (9, 4), (20, 6)])
def test_block_matches_library_formulation(layer, start, T):
    rng = np.random.default_rng(40 + start)
    q, k, v, g = _rand_layer_inputs(rng, T, layer)
    hs = max(0, start - layer.window + 1) if layer.window else 0
    k_hist = rng.standard_normal((start - hs, layer.hkv, layer.d))
    v_hist = rng.standard_normal((start - hs, layer.hkv, layer.d))
    y = oracle.block_bidirectional(q, k, v, g, k_hist, v_hist, hs, start, layer)
    ref = torch_block_reference(q, k, v, g, k_hist, v_hist, start, layer)
    assert np.allclose(y, ref, rtol=0, atol=1e-12)


def test_block_last_row_equals_causal_chunk_and_single_token_equals_decode():
    """The block's last row sees exactly what a causal chunk's last row sees;
    a one-token block is a decode step over the same history."""
    rng = np.random.default_rng(50)
    for layer in CHUNK_LAYERS:
        n, start = 18, 11
        q, k, v, g = _rand_layer_inputs(rng, n, layer)
        _, kh = oracle.qk_prologue(q, k, np.arange(n), layer)
        yb = oracle.block_bidirectional(q[start:], k[start:], v[start:], g[start:], kh[:start], v[:start], 0, start,
                                        layer)
        yc = oracle.prefill_chunk(q[start:], k[start:], v[start:], g[start:], kh[:start], v[:start], 0, start, layer)
        assert np.allclose(yb[-1], yc[-1], rtol=0, atol=1e-13)
        y1 = oracle.block_bidirectional(q[start:start + 1], k[start:start + 1], v[start:start + 1],
                                        g[start:start + 1], kh[:start], v[:start], 0, start, layer)
        yd = oracle.decode_one(q[start], k[start], v[start], g[start], kh[:start], v[:start], 0, start + 1, layer)
        assert np.allclose(y1[0], yd, rtol=0, atol=1e-13)


@pytest.mark.parametrize("mistake", ["causal", "one_sided_window"])
def test_planted_block_mistakes_fail_the_library_pin(mistake):
    """A causal mask, or a window without its forward edge, in place of the
    bidirectional window fails the library pin."""
    layer = CHUNK_LAYERS[0]                    # W = 6
    rng = np.random.default_rng(51)
    start, T = 9, 8                            # T > W: the forward window edge matters
    q, k, v, g = _rand_layer_inputs(rng, T, layer)
    hs = start - layer.window + 1
    k_hist = rng.standard_normal((start - hs, layer.hkv, layer.d))
    v_hist = rng.standard_normal((start - hs, layer.hkv, layer.d))
    ref = torch_block_reference(q, k, v, g, k_hist, v_hist, start, layer)
    assert np.allclose(oracle.block_bidirectional(q, k, v, g, k_hist, v_hist, hs, start, layer), ref,
                       rtol=0, atol=1e-12)
    if mistake == "causal":
        y = oracle.prefill_chunk(q, k, v, g, k_hist, v_hist, hs, start, layer)
    else:
        y = _block_one_sided(q, k, v, g, k_hist, v_hist, hs, start, layer)
    assert not np.allclose(y, ref, rtol=0, atol=1e-12)


def _block_one_sided(q, k, v, g, k_hist, v_hist, hs, start, layer):
    """The block attention with the forward window edge dropped (every later
    block key visible even beyond W): a plausible slip."""
    T = k.shape[0]
    pos = start + np.arange(T)
    qh = oracle.query_prologue(q, pos, layer)
    kh = oracle.key_prologue(k, pos, layer)
    keys = np.concatenate([k_hist, kh])
    vals = np.concatenate([v_hist, v])
    o = np.empty_like(qh)
    for t in range(T):
        lo = max(0, start + t - layer.window + 1) - hs
        w = oracle.softmax(oracle.logits_for_row(qh[t], keys[lo:], layer.group), axis=-1)
        for h in range(layer.hq):
            o[t, h] = w[h] @ vals[lo:, h // layer.group, :]
    return oracle.output_epilogue(o, g, layer)


# ---------------------------------------------------------------------------
# The flagged reference-rounding mode (reported beside the oracle, never the
# parity reference)
# ---------------------------------------------------------------------------

def test_to_bf16_rounds_to_nearest_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to the even one (1.0)
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 3.87, 5.4730064863875, -0.1, 65504.0, 1e-40])
    y = oracle.to_bf16(x)
    assert y[0] == 1.0 and y[1] == 1.0 and y[2] == 1.0 + 2.0 ** -6
    assert y[3] == 3.875 and y[4] == 5.46875            # bf16(3.87) and bf16(5.473...)
    assert abs(y[5] + 0.1) <= 2.0 ** -12 and y[6] == 65536.0
    # every result is a bf16 value: its float32 bits end in 16 zero bits
    assert np.all(y.astype(np.float32).view(np.uint32) & 0xFFFF == 0)


@pytest.mark.parametrize("scale,d", [(3.87, 128), (5.4730064863875, 64)])
def test_reference_rounding_moves_the_aligned_logit_to_the_rounded_multiplier(scale, d):
    """Aligned all-ones q and k: the plain oracle's logit is s * sqrt(d) * m / (m + 1e-5) with
    m = 1 (43.7836 on both models, the pages' eps figure); with the reference's casts the
    normalized entries round to 1 and the product q_hat * s to bf16, so the logit becomes
    bf16(s) * sqrt(d) (3.875 * sqrt(128) = 43.84; 5.46875 * 8 = 43.75)."""
    layer = Layer(hq=1, hkv=1, d=d, window=0, theta=0.0, scale=scale)
    ones = np.ones((1, 1, d))
    plain = oracle.logits_for_row(oracle.query_prologue(ones, [0], layer)[0],
                                  oracle.key_prologue(ones, [0], layer), 1)[0, 0]
    qr = oracle.query_prologue(ones, [0], layer, reference_rounding=True)
    kr = oracle.key_prologue(ones, [0], layer, reference_rounding=True)
    rounded = oracle.logits_for_row(qr[0], kr, 1)[0, 0]
    assert abs(plain - scale * np.sqrt(d) / (1 + 1e-5)) < 1e-12
    assert abs(rounded - oracle.to_bf16(scale)[()] * np.sqrt(d)) < 1e-12
    assert abs(rounded - plain) > 1e-2


def test_reference_rounding_stays_within_the_bf16_budget():
    """On N(0,1) inputs the flagged mode moves outputs by the bf16 rounding of q_hat,
    q_hat * s and k_hat only.  The logit error is about s * 2^-9 per unit, so each
    softmax weight moves by about 1 % and the largest of a few thousand outputs by a
    few 1e-2: more than the 2e-2 parity tolerance the GPU path meets with fp16
    operands, which is why the flagged mode is reported and never the reference."""
    rng = np.random.default_rng(70)
    for layer in (Layer(hq=8, hkv=2, d=64, window=16, theta=10000.0, scale=SPARK_SCALE, out_norm=True,
                        out_eps=1e-6),
                  Layer(hq=4, hkv=1, d=128, window=0, theta=0.0, scale=GLIMMER_SCALE)):
        T = 40
        q, k, v, g = _rand_layer_inputs(rng, T, layer)
        y = oracle.prefill(q, k, v, g, layer)
        yr = oracle.prefill(q, k, v, g, layer, reference_rounding=True)
        diff = np.max(np.abs(y - yr))
        assert 1e-3 < diff < 0.1
