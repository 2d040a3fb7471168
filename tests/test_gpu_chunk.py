"""GPU parity of chunked prefill (a chunk of T tokens continuing sequences
whose first start[b] positions are cached) against the fp64 oracle, through
the C ABI: outputs within the bf16 tolerance, and the cache afterwards holds
the chunk's keys (bf16 or E4M3 codes of the oracle's normalized and rotated
keys; a neighbouring code only where fp32 and fp64 fall on different sides
of a rounding midpoint) and values exactly, with every other entry as it
was."""
import numpy as np
import pytest
import torch

import global_muse_rope_amd as ma
import oracle
import synth
from oracle import fp8
from synth.workloads import Layer, GLIMMER_SCALE, SPARK_SCALE
from gpu_helpers import TOL, to_dev, max_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _f(bits):
    return synth.bf16_bits_to_f64(bits)


def make_chunk_cache(kind, layer, starts, T, page_tokens, use_fp8, seed=3, max_start=0, key_gain=None):
    """A cache holding each sequence's history before its chunk: a ring the
    last min(start, W) positions, a paged cache positions 0 .. start - 1 with
    pages mapped up to start + T - 1.  Returns the cache, the stored history
    as float64 [B, max_start, Hkv, D] (dequantized for E4M3), the host copies
    of k and v as stored, and the scales."""
    d, hkv, W = layer.d, layer.hkv, layer.window
    B = len(starts)
    maxs = max(1, int(max(starts)))
    n = B * maxs * hkv * d
    if use_fp8:
        kst = synth.e4m3_codes(seed, 40, np.arange(n)).reshape(B, maxs, hkv, d)
        vst = synth.e4m3_codes(seed, 41, np.arange(n)).reshape(B, maxs, hkv, d)
    else:
        kst = synth.normal_bf16_bits(seed, 40, (B, maxs, hkv, d))
        vst = synth.normal_bf16_bits(seed, 41, (B, maxs, hkv, d))
        if key_gain is not None:
            # cached keys of sequence b with RMS about key_gain[b] (stored as bf16)
            g = np.asarray(key_gain, dtype=np.float32)[:, None, None, None]
            kst = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(kst) * g)
    edt = np.uint8 if use_fp8 else np.uint16
    rng = np.random.default_rng(seed)
    if kind == "ring":
        kc = np.zeros((B, hkv, W, d), dtype=edt)
        vc = np.zeros((B, hkv, d, W), dtype=edt)
        ks = rng.uniform(0.05, 0.5, (B, hkv)).astype(np.float32)
        vs = rng.uniform(0.05, 0.5, (B, hkv)).astype(np.float32)
        for b, s in enumerate(starts):
            for p in range(max(0, s - W), s):
                kc[b, :, p % W, :] = kst[b, p]
                vc[b, :, :, p % W] = vst[b, p]
        table = None
        scale_of = lambda b, p: (ks[b], vs[b])                           # noqa: E731
    else:
        pt = page_tokens
        pages = (max(max(starts), max_start) + T + pt - 1) // pt
        n_pages = B * pages + 2
        table = np.random.default_rng(seed + 1).permutation(n_pages)[:B * pages].astype(np.int32).reshape(B, pages)
        kc = np.zeros((n_pages, hkv, pt, d), dtype=edt)
        vc = np.zeros((n_pages, hkv, d, pt), dtype=edt)
        ks = rng.uniform(0.05, 0.5, (n_pages, hkv)).astype(np.float32)
        vs = rng.uniform(0.05, 0.5, (n_pages, hkv)).astype(np.float32)
        for b, s in enumerate(starts):
            for p in range(s):
                kc[table[b, p // pt], :, p % pt, :] = kst[b, p]
                vc[table[b, p // pt], :, :, p % pt] = vst[b, p]
        scale_of = lambda b, p: (ks[table[b, p // pt]], vs[table[b, p // pt]])   # noqa: E731
    # the stored history as the oracle reads it
    hk = np.zeros((B, maxs, hkv, d))
    hv = np.zeros((B, maxs, hkv, d))
    for b, s in enumerate(starts):
        for p in range(s):
            if use_fp8:
                ksc, vsc = scale_of(b, p)
                hk[b, p] = fp8.dequantize(kst[b, p], ksc[:, None])
                hv[b, p] = fp8.dequantize(vst[b, p], vsc[:, None])
            else:
                hk[b, p] = _f(kst[b, p])
                hv[b, p] = _f(vst[b, p])

    def dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t if use_fp8 else t.view(torch.int16).view(torch.bfloat16)).to(DEV)

    kcs, vcs = (torch.from_numpy(ks).to(DEV), torch.from_numpy(vs).to(DEV)) if use_fp8 else (None, None)
    if kind == "ring":
        cache = ma.KvCache.ring(dev(kc), dev(vc), kcs, vcs)
    else:
        cache = ma.KvCache.paged(dev(kc), dev(vc), torch.from_numpy(table).to(DEV), page_tokens, kcs, vcs)
    return cache, hk, hv, kc, vc, ks, vs, table


def run_chunk_case(kind, layer, starts, T, page_tokens=32, use_fp8=False, max_start=None, bad=(), key_gain=None):
    B = len(starts)
    d = layer.d
    valid_starts = [s if b not in bad else 0 for b, s in enumerate(starts)]
    cache, hk, hv, kc0, vc0, ks, vs, table = make_chunk_cache(kind, layer, valid_starts, T, page_tokens, use_fp8,
                                                              max_start=max_start or 0, key_gain=key_gain)
    bits = {n: synth.normal_bf16_bits(7, sid, shp) for n, sid, shp in
            [("q", 1, (B, T, layer.hq, d)), ("k", 2, (B, T, layer.hkv, d)), ("v", 3, (B, T, layer.hkv, d)),
             ("g", 4, (B, T, layer.hq, d))]}
    dv = {n: to_dev(b) for n, b in bits.items()}
    max_start = int(max(valid_starts)) if max_start is None else max_start
    st = torch.tensor(starts, dtype=torch.int32, device=DEV)
    y = ma.prefill_chunk(ma.LayerParams.from_layer(layer), dv["q"], dv["k"], dv["v"], dv["g"], st, max_start,
                         cache)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    worst = 0.0
    for b, s in enumerate(starts):
        if b in bad:
            assert np.all(y[b] == 0)
            continue
        hs = max(0, s - layer.window + 1) if layer.window else 0
        ref = oracle.prefill_chunk(_f(bits["q"])[b], _f(bits["k"])[b], _f(bits["v"])[b], _f(bits["g"])[b],
                                   hk[b, hs:s], hv[b, hs:s], hs, s, layer)
        worst = max(worst, max_err(y[b], ref))
    print(f"chunk {kind} fp8={use_fp8} {layer} starts={starts} T={T} max_abs_err={worst:.3e}", flush=True)
    assert worst <= TOL
    check_cache_after(kind, layer, starts, T, bits, cache, kc0, vc0, ks, vs, table, page_tokens, use_fp8, bad)


# The device normalizes and rotates keys in fp32: an element carries an
# absolute error of a few fp32 ulps of the row's magnitude (about 1 after
# the norm), which decides the rounding of elements within that distance of
# a midpoint between two representable values.
KEY_ATOL = 4e-6


def _codes_close(got, x_scaled, vals, atol):
    """Each code's value lies within half its gap to the next code plus atol
    of x_scaled (the value the code rounds, computed in fp64)."""
    g = vals[got & 0x7F] * np.where(got & 0x80, -1.0, 1.0)
    mag = vals[got & 0x7F]
    gap = np.abs(vals[np.minimum((got & 0x7F).astype(int) + 1, 0x7E)] - mag)
    gap = np.maximum(gap, np.abs(mag - vals[np.maximum((got & 0x7F).astype(int) - 1, 0)]))
    assert np.all(np.abs(g - x_scaled) <= gap / 2 + atol)


def _bf16_close(got_bits, want_f64):
    """The stored bf16 lies within half a bf16 ulp plus KEY_ATOL of the fp64
    value (round to nearest of an fp32 value within KEY_ATOL of it)."""
    g = _f(got_bits)
    ulp = np.spacing(np.abs(g).astype(np.float32)).astype(np.float64) * 65536.0   # bf16 keeps 8 of fp32's 24 bits
    assert np.all(np.abs(g - want_f64) <= ulp / 2 + KEY_ATOL)


def check_cache_after(kind, layer, starts, T, bits, cache, kc0, vc0, ks, vs, table, pt, use_fp8, bad):
    W = layer.window
    kc = cache.k.cpu()
    vc = cache.v.cpu()
    kc = (kc if use_fp8 else kc.view(torch.int16)).numpy().view(np.uint8 if use_fp8 else np.uint16)
    vc = (vc if use_fp8 else vc.view(torch.int16)).numpy().view(np.uint8 if use_fp8 else np.uint16)
    expect_k = kc0.copy()
    expect_v = vc0.copy()
    written = np.zeros(kc0.shape[:3], dtype=bool)
    vals = fp8.e4m3_values()
    for b, s in enumerate(starts):
        if b in bad:
            continue
        pos = s + np.arange(T)
        kh = oracle.key_prologue(_f(bits["k"])[b], pos, layer)           # [T, Hkv, D]
        vraw = bits["v"][b]
        t_lo = max(0, T - W) if kind == "ring" else 0
        for t in range(t_lo, T):
            p = s + t
            if kind == "ring":
                loc = (b, slice(None), p % W)
                sk, sv = ks[b], vs[b]
            else:
                loc = (table[b, p // pt], slice(None), p % pt)
                sk, sv = ks[table[b, p // pt]], vs[table[b, p // pt]]
            got_k = kc[loc[0], :, loc[2], :]
            got_v = vc[loc[0], :, :, loc[2]]
            if use_fp8:
                _codes_close(got_k, kh[t] / sk[:, None], vals, KEY_ATOL / sk[:, None])
                assert np.array_equal(got_v, fp8.quantize(_f(vraw[t]), sv[:, None]))
            else:
                _bf16_close(got_k, kh[t])
                assert np.array_equal(got_v, vraw[t])
            written[loc[0], :, loc[2]] = True
    # every entry the chunk does not own is as it was
    keep = ~written
    assert np.array_equal(kc[keep], expect_k[keep])
    assert np.array_equal(np.moveaxis(vc, 3, 2)[keep], np.moveaxis(expect_v, 3, 2)[keep])


SPARK_SMALL = dict(hq=16, hkv=2, d=64, scale=SPARK_SCALE, out_norm=True, out_eps=1e-6)
GLIMMER_SMALL = dict(hq=32, hkv=2, d=128, scale=GLIMMER_SCALE)

CASES = [
    # (kind, layer, starts, T, page_tokens)
    ("paged", Layer(window=0, theta=0.0, **SPARK_SMALL), [0, 1, 63, 64, 100, 1000], 100, 32),
    ("paged", Layer(window=0, theta=0.0, **GLIMMER_SMALL), [0, 77, 300], 130, 16),
    ("ring", Layer(window=256, theta=10000.0, **SPARK_SMALL), [0, 5, 255, 256, 300, 1000], 100, 0),
    ("ring", Layer(window=256, theta=10000.0, **SPARK_SMALL), [0, 40, 700], 300, 0),       # T > W
    ("ring", Layer(window=128, theta=10000.0, **GLIMMER_SMALL), [0, 127, 500], 64, 0),
    ("paged", Layer(window=128, theta=10000.0, **SPARK_SMALL), [0, 200, 1000], 70, 32),   # windowed paged
]


@pytest.mark.parametrize("use_fp8", [False, True], ids=["bf16", "e4m3"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-d{c[1].d}w{c[1].window}T{c[3]}")
def test_prefill_chunk_parity(case, use_fp8):
    kind, layer, starts, T, pt = case
    run_chunk_case(kind, layer, starts, T, page_tokens=pt or 32, use_fp8=use_fp8)


def test_prefill_chunk_start_out_of_range():
    """start outside [0, max_start]: zero output, no cache write; the other
    sequences are unaffected."""
    layer = Layer(window=0, theta=0.0, **SPARK_SMALL)
    run_chunk_case("paged", layer, [50, -1, 30, 99], 40, page_tokens=32, max_start=64, bad=(1, 3))


@pytest.mark.parametrize("T", [200, 4200], ids=["key-split", "one-piece"])
def test_prefill_chunk_zero_start_matches_prefill(T):
    """With nothing cached the chunk is a whole-sequence prefill: bit for bit
    when the chunk launch has enough query blocks to run unsplit (T = 4200),
    and within one bf16 rounding when its few blocks are split over key
    pieces (T = 200), whose partial sums add in another order."""
    layer = Layer(window=256, theta=10000.0, **SPARK_SMALL)
    B = 2
    cache, *_ = make_chunk_cache("ring", layer, [0, 0], T, 32, False)
    bits = {n: synth.normal_bf16_bits(9, sid, shp) for n, sid, shp in
            [("q", 1, (B, T, 16, 64)), ("k", 2, (B, T, 2, 64)), ("v", 3, (B, T, 2, 64)), ("g", 4, (B, T, 16, 64))]}
    dv = {n: to_dev(b) for n, b in bits.items()}
    lp = ma.LayerParams.from_layer(layer)
    y1 = ma.prefill_chunk(lp, dv["q"], dv["k"], dv["v"], dv["g"], torch.zeros(B, dtype=torch.int32, device=DEV),
                          0, cache)
    y2 = ma.prefill(lp, dv["q"], dv["k"], dv["v"], dv["g"])
    torch.cuda.synchronize()
    if T > 1000:
        assert torch.equal(y1, y2)
    else:
        assert torch.allclose(y1.float(), y2.float(), rtol=2.0 ** -7, atol=1e-6)


# ---------------------------------------------------------------------------
# Non-causal drafter block over a cached context
# ---------------------------------------------------------------------------

def run_block_case(kind, layer, starts, T, page_tokens=32, use_fp8=False, key_gain=None):
    B = len(starts)
    d = layer.d
    cache, hk, hv, kc0, vc0, ks, vs, table = make_chunk_cache(kind, layer, starts, T, page_tokens, use_fp8,
                                                              key_gain=key_gain)
    bits = {n: synth.normal_bf16_bits(8, sid, shp) for n, sid, shp in
            [("q", 1, (B, T, layer.hq, d)), ("k", 2, (B, T, layer.hkv, d)), ("v", 3, (B, T, layer.hkv, d)),
             ("g", 4, (B, T, layer.hq, d))]}
    dv = {n: to_dev(b) for n, b in bits.items()}
    k_before = cache.k.clone()
    v_before = cache.v.clone()
    st = torch.tensor(starts, dtype=torch.int32, device=DEV)
    y = ma.draft_block(ma.LayerParams.from_layer(layer), dv["q"], dv["k"], dv["v"], dv["g"], st, int(max(starts)),
                       cache)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    worst = 0.0
    for b, s in enumerate(starts):
        hs = max(0, s - layer.window + 1) if layer.window else 0
        ref = oracle.block_bidirectional(_f(bits["q"])[b], _f(bits["k"])[b], _f(bits["v"])[b], _f(bits["g"])[b],
                                         hk[b, hs:s], hv[b, hs:s], hs, s, layer)
        worst = max(worst, max_err(y[b], ref))
    print(f"block {kind} fp8={use_fp8} {layer} starts={starts} T={T} max_abs_err={worst:.3e}", flush=True)
    assert worst <= TOL
    # the drafter's block is not kept: the cache is bit-for-bit unchanged
    assert torch.equal(cache.k, k_before) and torch.equal(cache.v, v_before)


BLOCK_CASES = [
    # (kind, layer, starts, T, page_tokens)
    ("ring", Layer(hq=32, hkv=8, d=128, window=2048, theta=10000.0, scale=GLIMMER_SCALE), [0, 5, 2047, 2048, 3000],
     16, 0),                                                                  # a 16-token drafter block
    ("paged", Layer(hq=128, hkv=16, d=64, window=2048, theta=10000.0, scale=SPARK_SCALE, out_norm=True,
                    out_eps=1e-6), [0, 700, 2600], 8, 32),                     # an 8-token block, windowed pages
    ("paged", Layer(window=0, theta=0.0, **SPARK_SMALL), [0, 1, 100, 1000], 16, 32),
    ("paged", Layer(window=0, theta=0.0, **SPARK_SMALL), [0, 63, 300], 150, 16),   # block wider than a tile
    ("ring", Layer(window=64, theta=10000.0, **SPARK_SMALL), [0, 30, 200], 100, 0),  # block wider than W
]


@pytest.mark.parametrize("use_fp8", [False, True], ids=["bf16", "e4m3"])
@pytest.mark.parametrize("case", BLOCK_CASES, ids=lambda c: f"{c[0]}-hq{c[1].hq}d{c[1].d}w{c[1].window}T{c[3]}")
def test_draft_block_parity(case, use_fp8):
    kind, layer, starts, T, pt = case
    run_block_case(kind, layer, starts, T, page_tokens=pt or 32, use_fp8=use_fp8)


# ---------------------------------------------------------------------------
# Cached keys above unit RMS
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("draft", [False, True], ids=["chunk", "block"])
@pytest.mark.parametrize("kind,window", [("ring", 256), ("paged", 0)])
def test_history_keys_above_unit_rms(kind, window, draft):
    """The cache is read as stored, so its key rows need not have RMS 1 (a
    cache written by other code, a mis-set E4M3 scale).  With RMS 1.5, 2 and
    2.5 the logits reach 95, 126 and 158 in log2 units, beyond what the
    max-free exponential takes unshifted; the outputs stay finite and within
    the tolerance of the oracle's max-subtracted softmax."""
    layer = Layer(window=window, theta=10000.0 if window else 0.0, **SPARK_SMALL)
    starts = [300, 700, 1000]
    gain = [1.5, 2.0, 2.5]
    if draft:
        run_block_case(kind, layer, starts, 16, page_tokens=32, key_gain=gain)
    else:
        run_chunk_case(kind, layer, starts, 100, page_tokens=32, key_gain=gain)


@pytest.mark.parametrize("kind,window", [("ring", 256), ("paged", 0)])
def test_few_token_block_keys_of_any_rms(kind, window):
    """A drafter block of at most 64 tokens keeps a running maximum over the
    cached keys, so keys of RMS 4 and 8 (logits bounded by about 250 and 500
    log2 units, beyond the fixed shift of the tile path) still give the
    oracle's max-subtracted softmax within the tolerance."""
    layer = Layer(window=window, theta=10000.0 if window else 0.0, **SPARK_SMALL)
    run_block_case(kind, layer, [300, 700, 1000], 16, page_tokens=32, key_gain=[4.0, 8.0, 1.0])
