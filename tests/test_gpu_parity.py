"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs.  Floating outputs: max-abs <= 2e-2 (bf16 outputs, fp32
accumulation).  Mask, ring and page logic: exact (test_*_visibility_exact)."""
import numpy as np
import pytest
import torch

import global_muse_rope_amd as ma
import oracle
import synth
from synth.workloads import Layer, GLIMMER_SCALE, SPARK_SCALE, TINY_LOCAL, TINY_GLOBAL
from gpu_helpers import TOL, to_dev, prefill_inputs_host, max_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _f(bits):
    return synth.bf16_bits_to_f64(bits)


def run_prefill(layer, bits, positions=None):
    d = {n: to_dev(b) for n, b in bits.items()}
    pos = torch.from_numpy(positions).to(DEV) if positions is not None else None
    y = ma.prefill(ma.LayerParams.from_layer(layer), d["q"], d["k"], d["v"], d["g"], positions=pos)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


def check_prefill(layer, B, T, seed=0, positions=None):
    bits = prefill_inputs_host(layer, B, T, seed)
    y = run_prefill(layer, bits, positions)
    worst = 0.0
    for b in range(B):
        pos = positions[b] if positions is not None else None
        ref = oracle.prefill(_f(bits["q"])[b], _f(bits["k"])[b], _f(bits["v"])[b], _f(bits["g"])[b], layer,
                             positions=pos)
        worst = max(worst, max_err(y[b], ref))
    print(f"{layer} B={B} T={T} max_abs_err={worst:.3e}", flush=True)
    assert worst <= TOL
    return worst


# ---------------------------------------------------------------------------
# Prologue
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,theta", [(64, 10000.0), (128, 10000.0), (128, 0.0), (64, 500000.0)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_rope_qknorm(d, theta, out_dtype):
    layer = Layer(hq=8, hkv=2, d=d, window=2048 if theta else 0, theta=theta, scale=SPARK_SCALE)
    n = 97
    qb = synth.normal_bf16_bits(5, 1, (n, 8, d))
    kb = synth.normal_bf16_bits(5, 2, (n, 2, d))
    pos = np.random.default_rng(0).integers(0, 1 << 20, size=n).astype(np.int32)
    pos[:4] = [0, 1, 262143, 1048575]
    qo, ko = ma.rope_qknorm(ma.LayerParams.from_layer(layer), to_dev(qb), to_dev(kb),
                            positions=torch.from_numpy(pos).to(DEV), out_dtype=out_dtype)
    torch.cuda.synchronize()
    rq = oracle.query_prologue(_f(qb), pos, layer)
    rk = oracle.key_prologue(_f(kb), pos, layer)
    rel = {torch.float32: 2e-6, torch.float16: 2 ** -10, torch.bfloat16: 2 ** -7}[out_dtype]
    for got, ref in ((qo, rq), (ko, rk)):
        g = got.float().cpu().numpy().astype(np.float64)
        assert np.all(np.abs(g - ref) <= rel * np.abs(ref) + 2e-5 * np.max(np.abs(ref)))


def test_rope_qknorm_strided_and_k_only():
    layer = Layer(hq=4, hkv=2, d=64, window=64, theta=10000.0, scale=3.0)
    n = 33
    fused = synth.normal_bf16_bits(6, 1, (n, 12, 64))      # [q(4) | k(2) | v(2) | g(4)] per token
    t = to_dev(fused)
    q = t[:, 0:4]
    k = t[:, 4:6]
    qo, ko = ma.rope_qknorm(ma.LayerParams.from_layer(layer), q, k)
    _, ko2 = ma.rope_qknorm(ma.LayerParams.from_layer(layer), None, k)
    torch.cuda.synchronize()
    f = _f(fused)
    rq = oracle.query_prologue(f[:, 0:4], np.arange(n), layer)
    rk = oracle.key_prologue(f[:, 4:6], np.arange(n), layer)
    assert max_err(qo.float().cpu().numpy(), rq) <= 2 ** -7 * np.max(np.abs(rq))
    assert max_err(ko.float().cpu().numpy(), rk) <= 2 ** -7 * np.max(np.abs(rk))
    assert torch.equal(ko, ko2)


# ---------------------------------------------------------------------------
# Prefill
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [TINY_LOCAL, TINY_GLOBAL], ids=lambda c: c.name)
def test_prefill_tiny_config_full(cfg):
    """The small configuration in full: 16 query heads on one KV head, D = 128,
    T = 1024, as a window-256 RoPE layer and as a global NoPE layer."""
    check_prefill(cfg.layer, cfg.batch, cfg.seq, cfg.seed)


@pytest.mark.parametrize("shape", [(16, 2, 64, 64, 10000.0, SPARK_SCALE, True, 300),
                                   (32, 2, 128, 256, 10000.0, GLIMMER_SCALE, False, 300)],
                         ids=["spark-like", "glimmer-like"])
def test_prefill_error_against_both_oracle_modes(shape):
    """Reports the GPU error against the oracle and against its flagged mode that
    rounds q_hat, q_hat * s and k_hat to bf16 as the pages' reference implementation
    does.  Parity is asserted against the oracle only; the second figure shows how far
    the reference's own casts sit from the GPU path (which keeps q_hat and k_hat in
    fp16, three more mantissa bits)."""
    hq, hkv, d, w, theta, scale, on, T = shape
    layer = Layer(hq=hq, hkv=hkv, d=d, window=w, theta=theta, scale=scale, out_norm=on, out_eps=1e-6)
    bits = prefill_inputs_host(layer, 1, T, 3)
    y = run_prefill(layer, bits)[0]
    args = (_f(bits["q"])[0], _f(bits["k"])[0], _f(bits["v"])[0], _f(bits["g"])[0], layer)
    ref = oracle.prefill(*args)
    ref_rounded = oracle.prefill(*args, reference_rounding=True)
    e_plain, e_rounded = max_err(y, ref), max_err(y, ref_rounded)
    print(f"{layer} T={T}: max_abs_err vs oracle {e_plain:.3e}, vs reference-rounding mode {e_rounded:.3e}, "
          f"reference-rounding mode vs oracle {max_err(ref_rounded, ref):.3e}", flush=True)
    assert e_plain <= TOL


SHAPES = [
    # (hq, hkv, d, window, theta, scale, out_norm, T)
    (16, 2, 64, 64, 10000.0, SPARK_SCALE, True, 300),      # Spark head shape, ragged T
    (16, 2, 64, 0, 0.0, SPARK_SCALE, True, 333),
    (32, 2, 128, 2048, 10000.0, GLIMMER_SCALE, False, 200),  # window larger than T
    (8, 8, 128, 17, 500000.0, GLIMMER_SCALE, False, 190),  # G = 1, odd window
    (8, 4, 64, 100, 10000.0, 2.5, True, 129),               # G = 2
    (16, 4, 128, 0, 0.0, GLIMMER_SCALE, True, 70),          # G = 4
    (16, 2, 128, 1, 10000.0, GLIMMER_SCALE, False, 65),     # window 1: self only
    (8, 1, 64, 0, 0.0, SPARK_SCALE, False, 1),              # a single token
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"hq{s[0]}kv{s[1]}d{s[2]}w{s[3]}T{s[7]}")
def test_prefill_shapes(shape):
    hq, hkv, d, w, th, s, on, T = shape
    layer = Layer(hq=hq, hkv=hkv, d=d, window=w, theta=th, scale=s, out_norm=on, out_eps=1e-6)
    check_prefill(layer, 1, T, seed=hq + T)


def test_prefill_batch_and_positions():
    layer = Layer(hq=16, hkv=2, d=64, window=50, theta=10000.0, scale=SPARK_SCALE, out_norm=True)
    B, T = 3, 150
    pos = np.stack([np.arange(T) + off for off in (0, 1000, 262000)]).astype(np.int32)
    check_prefill(layer, B, T, seed=3, positions=pos)


@pytest.mark.parametrize("T", [6001, 5000])
def test_prefill_local_many_blocks_per_workgroup(T):
    """A local layer with more query blocks than resident workgroups, so one
    workgroup walks several blocks in turn, loading each next block's queries
    ahead; two sequences, a ragged length and positions offset per sequence.
    At T = 5000 the 313 query blocks per head are padded to 320, so some of the
    blocks a workgroup loads ahead are padding.  Rows are sampled for the
    oracle (each row depends only on its own window)."""
    layer = Layer(hq=32, hkv=2, d=128, window=512, theta=10000.0, scale=GLIMMER_SCALE)
    B = 2
    pos = np.stack([np.arange(T), np.arange(T) + 70000]).astype(np.int32)
    bits = prefill_inputs_host(layer, B, T, seed=17)
    y = run_prefill(layer, bits, positions=pos)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(0, 20), np.arange(500, 530), np.arange(T - 40, T),
                                     rng.integers(0, T, 60)]))
    worst = 0.0
    for b in range(B):
        ref = oracle.prefill(_f(bits["q"])[b][rows], _f(bits["k"])[b][: rows.max() + 1],
                             _f(bits["v"])[b][: rows.max() + 1], _f(bits["g"])[b][rows], layer,
                             positions=pos[b], rows=rows)
        worst = max(worst, max_err(y[b][rows], ref))
    print(f"local many-blocks B={B} T={T} max_abs_err={worst:.3e}", flush=True)
    assert worst <= TOL


def test_prefill_strided_views():
    """q, k, v, gate as views of one fused [B, T, (Hq + 2 Hkv + Hq) * D] tensor;
    output written into a strided view."""
    layer = Layer(hq=8, hkv=2, d=128, window=40, theta=10000.0, scale=GLIMMER_SCALE)
    B, T = 2, 100
    fused = synth.normal_bf16_bits(4, 1, (B, T, 20, 128))
    t = to_dev(fused)
    q, k, v, g = t[:, :, 0:8], t[:, :, 8:10], t[:, :, 10:12], t[:, :, 12:20]
    big = torch.zeros((B, T, 10, 128), dtype=torch.bfloat16, device=DEV)
    out = big[:, :, 1:9]
    ma.prefill(ma.LayerParams.from_layer(layer), q, k, v, g, out=out)
    torch.cuda.synchronize()
    f = _f(fused)
    for b in range(B):
        ref = oracle.prefill(f[b, :, 0:8], f[b, :, 8:10], f[b, :, 10:12], f[b, :, 12:20], layer)
        assert max_err(out[b].float().cpu().numpy(), ref) <= TOL
    assert torch.count_nonzero(big[:, :, 0]) == 0 and torch.count_nonzero(big[:, :, 9]) == 0


@pytest.mark.parametrize("d,g,w", [(128, 16, 256), (64, 8, 2048), (64, 8, 0), (128, 16, 0), (64, 8, 100)])
def test_prefill_visibility_exact(d, g, w):
    """Exact mask check.  q = 0 makes every visible logit 0, so every visible
    key gets weight exactly 1/count; V is one-hot, dim c marking key m_c.  Then
    output dim c is nonzero iff key m_c is visible to the row: the visible set
    of every row is read off bit-exactly and compared with the oracle's
    visible_range."""
    hkv = 1
    T = 2300 if w == 2048 else 700
    layer = Layer(hq=g, hkv=hkv, d=d, window=w, theta=10000.0 if w else 0.0, scale=1.0)
    lp = ma.LayerParams.from_layer(layer)
    q = torch.zeros((1, T, g, d), dtype=torch.bfloat16, device=DEV)
    k = to_dev(synth.normal_bf16_bits(0, 2, (1, T, hkv, d)))
    gate = torch.full((1, T, g, d), 30.0, dtype=torch.bfloat16, device=DEV)
    rows = np.arange(T)
    for start in range(0, T, d):
        markers = np.arange(start, start + d)
        v = torch.zeros((1, T, hkv, d), dtype=torch.bfloat16, device=DEV)
        for c, m in enumerate(markers):
            if m < T:
                v[0, m, :, c] = 1.0
        y = ma.prefill(lp, q, k, v, gate)
        torch.cuda.synchronize()
        seen = (y[0].float().cpu().numpy() != 0)           # [T, g, d]
        lo = np.array([oracle.visible_range(i, w)[0] for i in rows])
        expect = (markers[None, :] >= lo[:, None]) & (markers[None, :] <= rows[:, None]) & (markers[None, :] < T)
        for h in range(g):
            assert np.array_equal(seen[:, h, :], expect), f"head {h} markers from {start}"


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------

def make_cache(kind, layer, B, lens, page_tokens=32, seed=1, dev=DEV):
    """Fill a ring or paged cache with stored entries for positions < L - 1 of
    each sequence; returns the cache and the per-sequence histories."""
    d, hkv = layer.d, layer.hkv
    maxL = int(max(lens))
    hist_k = synth.bf16_bits_to_f32(synth.normal_bf16_bits(seed, 10, (B, maxL, hkv, d)))
    hist_v = synth.bf16_bits_to_f32(synth.normal_bf16_bits(seed, 11, (B, maxL, hkv, d)))
    if kind == "ring":
        W = layer.window
        kc = torch.zeros((B, hkv, W, d), dtype=torch.bfloat16)
        vc = torch.zeros((B, hkv, d, W), dtype=torch.bfloat16)
        for b in range(B):
            L = int(lens[b])
            for p in range(max(0, L - 1 - W), L - 1):
                kc[b, :, p % W, :] = torch.from_numpy(hist_k[b, p])
                vc[b, :, :, p % W] = torch.from_numpy(hist_v[b, p])
        # the slot the new token will take holds a stale entry (position L-1-W)
        return ma.KvCache.ring(kc.to(dev), vc.to(dev)), hist_k, hist_v
    pages_per = (maxL + page_tokens - 1) // page_tokens
    n_pages = B * pages_per + 3
    perm = np.random.default_rng(seed).permutation(n_pages)[: B * pages_per].astype(np.int32)
    table = perm.reshape(B, pages_per)
    kc = torch.zeros((n_pages, hkv, page_tokens, d), dtype=torch.bfloat16)
    vc = torch.zeros((n_pages, hkv, d, page_tokens), dtype=torch.bfloat16)
    for b in range(B):
        L = int(lens[b])
        for p in range(L - 1):
            pg, r = table[b, p // page_tokens], p % page_tokens
            kc[pg, :, r, :] = torch.from_numpy(hist_k[b, p])
            vc[pg, :, :, r] = torch.from_numpy(hist_v[b, p])
    cache = ma.KvCache.paged(kc.to(dev), vc.to(dev), torch.from_numpy(table).to(dev), page_tokens)
    return cache, hist_k, hist_v


DEC_CASES = [
    # (kind, hq, hkv, d, window, theta, scale, out_norm, lens, page_tokens)
    ("paged", 16, 2, 64, 0, 0.0, SPARK_SCALE, True, [300, 77, 1, 2, 33, 64], 32),
    ("paged", 32, 2, 128, 0, 0.0, GLIMMER_SCALE, False, [5000, 4097, 4096, 17], 16),
    ("ring", 16, 2, 64, 256, 10000.0, SPARK_SCALE, True, [1, 2, 255, 256, 257, 1000], 0),
    ("ring", 32, 2, 128, 64, 10000.0, GLIMMER_SCALE, False, [63, 64, 65, 129, 3], 0),
    ("paged", 16, 2, 64, 128, 10000.0, SPARK_SCALE, True, [500, 128, 129, 3000], 32),   # local layer, paged
]


@pytest.mark.parametrize("case", DEC_CASES, ids=lambda c: f"{c[0]}-hq{c[1]}d{c[3]}w{c[4]}")
def test_decode_parity(case):
    kind, hq, hkv, d, w, th, s, on, lens, pt = case
    layer = Layer(hq=hq, hkv=hkv, d=d, window=w, theta=th, scale=s, out_norm=on, out_eps=1e-6)
    B = len(lens)
    lens = np.array(lens, dtype=np.int32)
    cache, hk, hv = make_cache(kind, layer, B, lens, page_tokens=pt or 32)
    new = {n: synth.normal_bf16_bits(2, sid, shp) for n, sid, shp in
           [("q", 12, (B, hq, d)), ("k", 13, (B, hkv, d)), ("v", 14, (B, hkv, d)), ("g", 15, (B, hq, d))]}
    dn = {n: to_dev(b) for n, b in new.items()}
    kv = torch.from_numpy(lens).to(DEV)
    out = ma.decode(ma.LayerParams.from_layer(layer), dn["q"], dn["k"], dn["v"], dn["g"], kv, int(lens.max()), cache)
    torch.cuda.synchronize()
    y = out.float().cpu().numpy()
    worst = 0.0
    for b in range(B):
        L = int(lens[b])
        fb = {n: _f(v)[b] for n, v in new.items()}
        ref = oracle.decode_one(fb["q"], fb["k"], fb["v"], fb["g"], hk[b, :max(L - 1, 0)].astype(np.float64),
                                hv[b, :max(L - 1, 0)].astype(np.float64), 0, L, layer)
        worst = max(worst, max_err(y[b], ref))
    print(f"decode {case} max_abs_err={worst:.3e}", flush=True)
    assert worst <= TOL
    # the new entry was written into the cache, key normalized (+ rotated) and value as given
    kh_new = oracle.key_prologue(_f(new["k"]), np.maximum(lens - 1, 0), layer)  # [B, Hkv, D], one position per row
    for b in range(B):
        p = int(lens[b]) - 1
        if kind == "ring":
            kst = cache.k[b, :, p % w, :].float().cpu().numpy()
            vst = cache.v[b, :, :, p % w].float().cpu().numpy()
        else:
            pg = int(cache.block_table[b, p // pt])
            kst = cache.k[pg, :, p % pt, :].float().cpu().numpy()
            vst = cache.v[pg, :, :, p % pt].float().cpu().numpy()
        assert np.allclose(kst, kh_new[b], rtol=2 ** -8, atol=1e-6)
        assert np.array_equal(vst, synth.bf16_bits_to_f32(new["v"][b]))


@pytest.mark.parametrize("kind,w", [("ring", 64), ("paged", 0), ("paged", 48)])
def test_decode_visibility_exact(kind, w):
    """Exact check of the ring slots and page walk: q = 0 gives every visible
    entry weight 1/count; cached V is one-hot by position (dim c marks position
    m_c), the new token's v is zero.  Output dim c is nonzero iff position m_c
    is visible."""
    d, hkv, hq = 64, 1, 8
    layer = Layer(hq=hq, hkv=hkv, d=d, window=w, theta=10000.0 if w else 0.0, scale=1.0)
    lens = np.array([1, 2, 63, 64, 65, 100, 130, 200], dtype=np.int32)
    B = len(lens)
    maxL = int(lens.max())
    for start in range(0, maxL, d):
        markers = np.arange(start, start + d)
        if kind == "ring":
            kc = torch.zeros((B, hkv, w, d), dtype=torch.bfloat16)
            vc = torch.zeros((B, hkv, d, w), dtype=torch.bfloat16)
            for b in range(B):
                L = int(lens[b])
                for p in range(max(0, L - 1 - w), L - 1):
                    c = p - start
                    if 0 <= c < d:
                        vc[b, :, c, p % w] = 1.0
                # the slot the new token takes holds a stale marker: it must stay invisible
                p = L - 1 - w
                if p >= 0 and 0 <= p - start < d:
                    vc[b, :, p - start, p % w] = 1.0
            cache = ma.KvCache.ring(kc.to(DEV), vc.to(DEV))
        else:
            pt = 16
            pages_per = (maxL + pt - 1) // pt
            table = np.random.default_rng(start).permutation(B * pages_per).astype(np.int32).reshape(B, pages_per)
            kc = torch.zeros((B * pages_per, hkv, pt, d), dtype=torch.bfloat16)
            vc = torch.zeros((B * pages_per, hkv, d, pt), dtype=torch.bfloat16)
            for b in range(B):
                L = int(lens[b])
                for p in range(pages_per * pt):
                    c = p - start
                    if 0 <= c < d and p != L - 1:
                        vc[table[b, p // pt], :, c, p % pt] = 1.0   # markers also beyond L: must stay invisible
            cache = ma.KvCache.paged(kc.to(DEV), vc.to(DEV), torch.from_numpy(table).to(DEV), pt)
        q = torch.zeros((B, hq, d), dtype=torch.bfloat16, device=DEV)
        kn = to_dev(synth.normal_bf16_bits(0, 13, (B, hkv, d)))
        vn = torch.zeros((B, hkv, d), dtype=torch.bfloat16, device=DEV)
        g = torch.full((B, hq, d), 30.0, dtype=torch.bfloat16, device=DEV)
        out = ma.decode(ma.LayerParams.from_layer(layer), q, kn, vn, g, torch.from_numpy(lens).to(DEV),
                        maxL, cache)
        torch.cuda.synchronize()
        seen = out.float().cpu().numpy() != 0
        for b in range(B):
            L = int(lens[b])
            lo, hi = oracle.visible_range(L - 1, w)
            expect = (markers >= lo) & (markers <= hi - 1)      # cached positions only (new v is zero)
            for h in range(hq):
                assert np.array_equal(seen[b, h], expect), (b, L, start)


@pytest.mark.parametrize("kind,w,d,lens", [
    ("paged", 0, 64, [300, 77, 1, 2, 33, 64, 17]),
    ("ring", 256, 64, [1, 2, 9, 100, 255]),
    ("paged", 0, 128, [5000, 17, 40]),
])
def test_decode_unwritten_entries_ignored(kind, w, d, lens):
    """Cache entries never written (ring slots and page rows at or past the
    sequence's last position, and unused pages) may hold any bits: poisoned
    with NaN they must leave the output bit-identical to zero-filled ones."""
    hq, hkv = (16, 2) if d == 64 else (32, 2)
    layer = Layer(hq=hq, hkv=hkv, d=d, window=w, theta=10000.0 if w else 0.0,
                  scale=SPARK_SCALE, out_norm=(d == 64), out_eps=1e-6)
    B = len(lens)
    lens = np.array(lens, dtype=np.int32)
    new = {n: to_dev(synth.normal_bf16_bits(3, sid, shp)) for n, sid, shp in
           [("q", 12, (B, hq, d)), ("k", 13, (B, hkv, d)), ("v", 14, (B, hkv, d)), ("g", 15, (B, hq, d))]}
    kv = torch.from_numpy(lens).to(DEV)
    outs = []
    for poison in (False, True):
        cache, _, _ = make_cache(kind, layer, B, lens, page_tokens=16)
        if poison:
            k, v = cache.k, cache.v
            if kind == "ring":
                for b in range(B):
                    L = int(lens[b])
                    if L - 1 < w:
                        k[b, :, L - 1:, :] = float("nan")
                        v[b, :, :, L - 1:] = float("nan")
            else:
                table = cache.block_table.cpu().numpy()
                used = set()
                for b in range(B):
                    L = int(lens[b])
                    for p in range(table.shape[1] * 16):
                        pg, r = int(table[b, p // 16]), p % 16
                        if p < L - 1:
                            used.add((pg, r))
                for pg in range(k.shape[0]):
                    for r in range(16):
                        if (pg, r) not in used:
                            k[pg, :, r, :] = float("nan")
                            v[pg, :, :, r] = float("nan")
        y = ma.decode(ma.LayerParams.from_layer(layer), new["q"], new["k"], new["v"], new["g"], kv,
                      int(lens.max()), cache)
        torch.cuda.synchronize()
        outs.append(y.float().cpu())
    assert torch.isfinite(outs[1]).all()
    assert torch.equal(outs[0], outs[1])


# ---------------------------------------------------------------------------
# Decode over an FP8 (E4M3) cache
# ---------------------------------------------------------------------------

def make_cache_fp8(kind, layer, B, lens, page_tokens=32, seed=1, dev=DEV):
    """Like make_cache, with entries stored as E4M3 codes of value / scale
    (the oracle's quantizer) and seeded per-(page, head) or per-(sequence,
    head) scales.  Returns the cache and the dequantized histories."""
    from oracle import fp8
    d, hkv = layer.d, layer.hkv
    maxL = int(max(lens))
    hist_k = synth.bf16_bits_to_f32(synth.normal_bf16_bits(seed, 10, (B, maxL, hkv, d)))
    hist_v = synth.bf16_bits_to_f32(synth.normal_bf16_bits(seed, 11, (B, maxL, hkv, d)))
    rng = np.random.default_rng(seed + 100)
    if kind == "ring":
        W = layer.window
        ks = rng.uniform(0.02, 0.5, (B, hkv)).astype(np.float32)
        vs = rng.uniform(0.02, 0.5, (B, hkv)).astype(np.float32)
        kc = np.zeros((B, hkv, W, d), dtype=np.uint8)
        vc = np.zeros((B, hkv, d, W), dtype=np.uint8)
        dk = np.zeros_like(hist_k, dtype=np.float64)
        dv = np.zeros_like(hist_v, dtype=np.float64)
        for b in range(B):
            L = int(lens[b])
            for p in range(max(0, L - 1 - W), L - 1):
                for h in range(hkv):
                    kc[b, h, p % W] = fp8.quantize(hist_k[b, p, h], ks[b, h])
                    vc[b, h, :, p % W] = fp8.quantize(hist_v[b, p, h], vs[b, h])
                    dk[b, p, h] = fp8.dequantize(kc[b, h, p % W], ks[b, h])
                    dv[b, p, h] = fp8.dequantize(vc[b, h, :, p % W], vs[b, h])
        cache = ma.KvCache.ring(torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev),
                                torch.from_numpy(ks).to(dev), torch.from_numpy(vs).to(dev))
        return cache, dk, dv, ks, vs
    pages_per = (maxL + page_tokens - 1) // page_tokens
    n_pages = B * pages_per + 3
    perm = np.random.default_rng(seed).permutation(n_pages)[: B * pages_per].astype(np.int32)
    table = perm.reshape(B, pages_per)
    ks = rng.uniform(0.02, 0.5, (n_pages, hkv)).astype(np.float32)
    vs = rng.uniform(0.02, 0.5, (n_pages, hkv)).astype(np.float32)
    kc = np.zeros((n_pages, hkv, page_tokens, d), dtype=np.uint8)
    vc = np.zeros((n_pages, hkv, d, page_tokens), dtype=np.uint8)
    dk = np.zeros_like(hist_k, dtype=np.float64)
    dv = np.zeros_like(hist_v, dtype=np.float64)
    for b in range(B):
        L = int(lens[b])
        for p in range(L - 1):
            pg, r = table[b, p // page_tokens], p % page_tokens
            for h in range(hkv):
                kc[pg, h, r] = fp8.quantize(hist_k[b, p, h], ks[pg, h])
                vc[pg, h, :, r] = fp8.quantize(hist_v[b, p, h], vs[pg, h])
                dk[b, p, h] = fp8.dequantize(kc[pg, h, r], ks[pg, h])
                dv[b, p, h] = fp8.dequantize(vc[pg, h, :, r], vs[pg, h])
    cache = ma.KvCache.paged(torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev),
                             torch.from_numpy(table).to(dev), page_tokens,
                             torch.from_numpy(ks).to(dev), torch.from_numpy(vs).to(dev))
    return cache, dk, dv, ks, vs


FP8_CASES = [
    # (kind, hq, hkv, d, window, theta, scale, out_norm, lens, page_tokens)
    ("paged", 16, 2, 64, 0, 0.0, SPARK_SCALE, True, [300, 77, 1, 2, 33, 64], 32),
    ("paged", 32, 2, 128, 0, 0.0, GLIMMER_SCALE, False, [1500, 513, 17], 16),
    ("ring", 16, 2, 64, 256, 10000.0, SPARK_SCALE, True, [1, 2, 255, 256, 257, 700], 0),
    ("paged", 16, 2, 64, 128, 10000.0, SPARK_SCALE, True, [500, 128, 129], 32),
]


@pytest.mark.parametrize("case", FP8_CASES, ids=lambda c: f"{c[0]}-hq{c[1]}d{c[3]}w{c[4]}")
def test_decode_fp8_parity(case):
    """Decode over E4M3 codes against the oracle on the dequantized cache; the
    new entry's codes against the oracle's quantizer."""
    from oracle import fp8
    kind, hq, hkv, d, w, th, s, on, lens, pt = case
    layer = Layer(hq=hq, hkv=hkv, d=d, window=w, theta=th, scale=s, out_norm=on, out_eps=1e-6)
    B = len(lens)
    lens = np.array(lens, dtype=np.int32)
    cache, dk, dv, ks, vs = make_cache_fp8(kind, layer, B, lens, page_tokens=pt or 32)
    new = {n: synth.normal_bf16_bits(2, sid, shp) for n, sid, shp in
           [("q", 12, (B, hq, d)), ("k", 13, (B, hkv, d)), ("v", 14, (B, hkv, d)), ("g", 15, (B, hq, d))]}
    dn = {n: to_dev(b) for n, b in new.items()}
    kv = torch.from_numpy(lens).to(DEV)
    out = ma.decode(ma.LayerParams.from_layer(layer), dn["q"], dn["k"], dn["v"], dn["g"], kv, int(lens.max()), cache)
    torch.cuda.synchronize()
    y = out.float().cpu().numpy()
    worst = 0.0
    for b in range(B):
        L = int(lens[b])
        fb = {n: _f(v)[b] for n, v in new.items()}
        ref = oracle.decode_one(fb["q"], fb["k"], fb["v"], fb["g"], dk[b, :max(L - 1, 0)], dv[b, :max(L - 1, 0)],
                                0, L, layer)
        worst = max(worst, max_err(y[b], ref))
    print(f"decode fp8 {case} max_abs_err={worst:.3e}", flush=True)
    assert worst <= TOL
    # the new entry's codes: values exactly; keys exactly except where the
    # fp32 and fp64 normalized keys fall on different sides of a rounding
    # midpoint (then the codes are neighbours)
    kh_new = oracle.key_prologue(_f(new["k"]), np.maximum(lens - 1, 0), layer)
    kc = cache.k.cpu().numpy()
    vc = cache.v.cpu().numpy()
    table = cache.block_table.cpu().numpy() if kind == "paged" else None
    vals = fp8.e4m3_values()
    for b in range(B):
        p = int(lens[b]) - 1
        for h in range(hkv):
            if kind == "ring":
                kst, vst, si = kc[b, h, p % w], vc[b, h, :, p % w], (b, h)
            else:
                pg = int(table[b, p // pt])
                kst, vst, si = kc[pg, h, p % pt], vc[pg, h, :, p % pt], (pg, h)
            assert np.array_equal(vst, fp8.quantize(_f(new["v"])[b, h], vs[si]))
            want = fp8.quantize(kh_new[b, h], ks[si])
            diff = want != kst
            if diff.any():
                x = (kh_new[b, h].astype(np.float32) / ks[si])[diff].astype(np.float64)
                mid = (vals[want[diff] & 0x7F] + vals[kst[diff] & 0x7F]) / 2 * np.sign(x)
                assert np.all(np.abs(np.abs(want[diff].astype(int) & 0x7F) - (kst[diff].astype(int) & 0x7F)) == 1)
                assert np.allclose(x, mid, rtol=1e-5), (b, h, x, mid)


def test_decode_fp8_value_codes_exact():
    """Every finite E4M3 code read back exactly: one cached entry, q = 0 (equal
    weights), v_new = 0 and a gate of 30 (sigmoid 1 in fp32), so each output
    is value(code) * scale / 2, exact in bf16 for power-of-two scales."""
    from oracle import fp8
    d, hkv, hq = 64, 4, 8
    layer = Layer(hq=hq, hkv=hkv, d=d, window=0, theta=0.0, scale=1.0)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    B = (len(codes) + hkv * d - 1) // (hkv * d)
    vcodes = np.resize(codes, (B, hkv, d)).astype(np.uint8)
    pt = 16
    table = np.arange(B, dtype=np.int32).reshape(B, 1)
    kc = np.zeros((B, hkv, pt, d), dtype=np.uint8)
    vc = np.zeros((B, hkv, d, pt), dtype=np.uint8)
    vc[:, :, :, 0] = vcodes
    ks = np.ones((B, hkv), dtype=np.float32)
    vs = np.full((B, hkv), 4.0, dtype=np.float32)
    cache = ma.KvCache.paged(torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV),
                             torch.from_numpy(table).to(DEV), pt, torch.from_numpy(ks).to(DEV),
                             torch.from_numpy(vs).to(DEV))
    q = torch.zeros((B, hq, d), dtype=torch.bfloat16, device=DEV)
    kn = to_dev(synth.normal_bf16_bits(0, 13, (B, hkv, d)))
    vn = torch.zeros((B, hkv, d), dtype=torch.bfloat16, device=DEV)
    g = torch.full((B, hq, d), 30.0, dtype=torch.bfloat16, device=DEV)
    lens = torch.full((B,), 2, dtype=torch.int32, device=DEV)
    y = ma.decode(ma.LayerParams.from_layer(layer), q, kn, vn, g, lens, 2, cache)
    torch.cuda.synchronize()
    want = fp8.e4m3_decode(vcodes) * 4.0 / 2.0                 # [B, Hkv, D]
    got = y.float().cpu().numpy().reshape(B, hkv, hq // hkv, d)
    for j in range(hq // hkv):
        assert np.array_equal(got[:, :, j, :], want)
