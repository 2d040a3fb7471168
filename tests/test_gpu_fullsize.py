"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (caller-provided output and workspace, default strides).

The oracle cannot finish a whole 32K-262K-token layer in seconds, so each
test compares sampled outputs: every query head of a few KV-head groups, on
rows that cover the first tile, tile and window edges, the last rows and a
seeded random set.  Each output row depends only on its own query and its
visible keys, so a sampled row is checked exactly as in a full run.  KV-head
groups are independent (grouped-query attention), so the oracle runs one
group at a time as a layer with G query heads and one KV head.  Properties
that hold at any size (every output finite; without the output norm,
|y| <= max |v| over the visible values of the head's group) are checked on
all outputs.  Decode checks sampled (sequence, KV head) pairs of the paged
global cache and every pair of the local ring.
"""
import dataclasses
import time

import numpy as np
import pytest
import torch

import global_muse_rope_amd as ma
import oracle
from synth import device as sd
from synth import workloads as wl
from gpu_helpers import TOL, max_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def sample_rows(T, W, seed=1, n_random=8):
    rows = {0, 1, 2, 3, 63, 64, 65, 127, 128, 129, T - 65, T - 64, T - 2, T - 1}
    if W:
        rows |= {W - 2, W - 1, W, W + 1}
    rows |= set(np.random.default_rng(seed).integers(0, T, size=n_random).tolist())
    return sorted(r for r in rows if 0 <= r < T)


def group_layer(layer):
    """The layer restricted to one KV-head group (G query heads, 1 KV head)."""
    return dataclasses.replace(layer, hq=layer.group, hkv=1)


def oracle_group_rows(cfg, hk, rows):
    """fp64 oracle outputs [n_rows, G, D] of query heads hk*G .. hk*G+G-1."""
    L = cfg.layer
    G = L.group
    gl = group_layer(L)
    heads = np.arange(hk * G, (hk + 1) * G)
    q = sd.host_rows(cfg, "q", 0, rows, heads)
    g = sd.host_rows(cfg, "g", 0, rows, heads)
    out = np.empty((len(rows), G, L.d))
    if L.window:
        # local layer: only the W keys ending at the row are visible; pass that
        # slice with its absolute positions (RoPE uses positions, visibility
        # uses indices within the slice, which start at the window's start)
        for n, i in enumerate(rows):
            t0 = max(0, i - L.window + 1)
            k = sd.host_tokens(cfg, "k", 0, t0, i + 1, [hk])
            v = sd.host_tokens(cfg, "v", 0, t0, i + 1, [hk])
            out[n] = oracle.prefill(q[n:n + 1], k, v, g[n:n + 1], gl,
                                    positions=np.arange(t0, i + 1), rows=[i - t0])[0]
        return out
    top = max(rows) + 1
    k = sd.host_tokens(cfg, "k", 0, 0, top, [hk])
    v = sd.host_tokens(cfg, "v", 0, 0, top, [hk])
    return oracle.prefill(q, k, v, g, gl, rows=rows)


PREFILL_FULL = [wl.GLIMMER_LOCAL, wl.GLIMMER_GLOBAL, wl.SPARK_LOCAL, wl.SPARK_GLOBAL]


@pytest.mark.parametrize("cfg", PREFILL_FULL, ids=lambda c: c.name)
def test_prefill_fullsize_sampled(cfg):
    L = cfg.layer
    print(f"prefill full size {cfg.name}", flush=True)
    lp = ma.LayerParams.from_layer(L)
    x = sd.prefill_device_inputs(cfg)
    out = torch.empty((cfg.batch, cfg.seq, L.hq, L.d), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(ma.prefill_workspace_size(lp, cfg.batch, cfg.seq), dtype=torch.uint8, device=DEV)
    ma.prefill(lp, x["q"], x["k"], x["v"], x["g"], out=out, workspace=ws)
    torch.cuda.synchronize()

    # properties over every output
    assert bool(torch.isfinite(out).all())
    if not L.out_norm:
        # o is a convex combination of visible values and sigma(g) < 1; the
        # running maximum of |v| over tokens bounds every row (bf16 slack)
        vabs = x["v"][0].abs().float()                                  # [T, Hkv, D]
        vmax = torch.cummax(vabs, dim=0).values                         # [T, Hkv, D]
        bound = vmax.repeat_interleave(L.group, dim=1) * (1 + 2 ** -7) + 1e-6
        assert bool((out[0].abs().float() <= bound).all())
        del vabs, vmax, bound
    del ws, x
    torch.cuda.empty_cache()

    # local rows are cheap (W keys each): more rows and every group
    rows = sample_rows(cfg.seq, L.window, n_random=32 if L.window else 16)
    groups = range(L.hkv) if L.window else sorted({0, L.hkv - 1})
    worst = 0.0
    t = time.time()
    for hk in groups:
        ref = oracle_group_rows(cfg, hk, rows)
        y = out[0, rows, hk * L.group:(hk + 1) * L.group].float().cpu().numpy()
        worst = max(worst, max_err(y, ref))
    print(f"{cfg.name}: {len(rows)} rows x {len(groups) * L.group} heads, max_abs_err={worst:.3e} "
          f"(oracle {time.time() - t:.1f} s)", flush=True)
    assert worst <= TOL


def _decode_run(cfg, fp8=False, lengths=None):
    L = cfg.layer
    s = sd.decode_device_setup(cfg, fp8=fp8, lengths=lengths)
    ks, vs = s.get("k_scale"), s.get("v_scale")
    if s["kind"] == "ring":
        cache = ma.KvCache.ring(s["kc"], s["vc"], ks, vs)
    else:
        cache = ma.KvCache.paged(s["kc"], s["vc"], s["block_table"], s["page_tokens"], ks, vs)
    lp = ma.LayerParams.from_layer(L)
    ws = torch.empty(ma.decode_workspace_size(lp, cfg.batch, s["max_len"], cache), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty((cfg.batch, L.hq, L.d), dtype=torch.bfloat16, device=DEV)
    ma.decode(lp, s["q"], s["k"], s["v"], s["g"], s["kv_len"], s["max_len"], cache, out=out, workspace=ws)
    torch.cuda.synchronize()
    y = out.float().cpu().numpy()
    lengths = s["lengths"]
    extra = {k: s[k] for k in ("scales_host", "table_host", "page_tokens") if k in s}
    del s, cache, ws, out
    torch.cuda.empty_cache()
    if fp8:
        return y, lengths, extra
    return y, lengths


def oracle_decode_pair(cfg, new, b, hk, L_b):
    """fp64 oracle output [G, D] of sequence b, KV head hk's query heads."""
    lay = cfg.layer
    G = lay.group
    p = L_b - 1
    lo, _ = oracle.visible_range(p, lay.window)
    k_hist = sd.cache_values_host(cfg.seed, b, hk, lay.hkv, "k", lo, p, lay.d)[:, None, :]
    v_hist = sd.cache_values_host(cfg.seed, b, hk, lay.hkv, "v", lo, p, lay.d)[:, None, :]
    hs = slice(hk * G, (hk + 1) * G)
    return oracle.decode_one(new["q"][b, hs], new["k"][b, hk:hk + 1], new["v"][b, hk:hk + 1], new["g"][b, hs],
                             k_hist, v_hist, lo, L_b, group_layer(lay))


def paged_pairs(lengths, hkv):
    """(sequence, KV head) pairs checked on the paged workload: the two
    shortest sequences and the two longest (near 2^20 positions: about 122
    chunks of 8192 entries, 7-8 chunks per combine wave), two or more KV heads
    of each, the first and last heads among them."""
    order = np.argsort(lengths)
    return [(int(order[0]), 0), (int(order[0]), hkv - 1), (int(order[1]), 5),
            (int(order[-1]), 0), (int(order[-1]), hkv - 1), (int(order[-2]), 3), (int(order[-2]), 10)]


def test_decode_fullsize_global_paged_sampled():
    cfg = wl.SPARK_DECODE_GLOBAL
    print(f"decode full size {cfg.name}", flush=True)
    y, lengths = _decode_run(cfg)
    assert np.isfinite(y).all()
    new = sd.new_token_host(cfg)
    pairs = paged_pairs(lengths, cfg.layer.hkv)
    worst = 0.0
    t = time.time()
    for b, hk in pairs:
        ref = oracle_decode_pair(cfg, new, b, hk, int(lengths[b]))
        G = cfg.layer.group
        worst = max(worst, max_err(y[b, hk * G:(hk + 1) * G], ref))
    print(f"{cfg.name}: pairs {pairs} lengths {[int(lengths[b]) for b, _ in pairs]} "
          f"max_abs_err={worst:.3e} (oracle {time.time() - t:.1f} s)", flush=True)
    assert worst <= TOL


def test_decode_fullsize_local_ring_all():
    cfg = wl.SPARK_DECODE_LOCAL
    print(f"decode full size {cfg.name}", flush=True)
    y, lengths = _decode_run(cfg)
    new = sd.new_token_host(cfg)
    G = cfg.layer.group
    worst = 0.0
    for b in range(cfg.batch):
        for hk in range(cfg.layer.hkv):
            ref = oracle_decode_pair(cfg, new, b, hk, int(lengths[b]))
            worst = max(worst, max_err(y[b, hk * G:(hk + 1) * G], ref))
    print(f"{cfg.name}: all {cfg.batch * cfg.layer.hkv} pairs, max_abs_err={worst:.3e}", flush=True)
    assert worst <= TOL


def oracle_decode_pair_fp8(cfg, new, b, hk, L_b, extra):
    """As oracle_decode_pair over an E4M3 cache: the history is the codes
    regenerated on the host, dequantized with each position's scale (page
    of the block table, or the sequence's scale for a ring)."""
    from oracle import fp8
    lay = cfg.layer
    G = lay.group
    p = L_b - 1
    lo, _ = oracle.visible_range(p, lay.window)
    ks, vs = extra["scales_host"]
    pos = np.arange(lo, p)
    if "table_host" in extra:
        pages = extra["table_host"][b, pos // extra["page_tokens"]]
        k_sc, v_sc = ks[pages, hk], vs[pages, hk]
    else:
        k_sc = np.full(len(pos), ks[b, hk], dtype=np.float32)
        v_sc = np.full(len(pos), vs[b, hk], dtype=np.float32)
    hist = {}
    for which, sc in (("k", k_sc), ("v", v_sc)):
        codes = sd.cache_codes_host(cfg.seed, b, hk, lay.hkv, which, lo, p, lay.d)
        hist[which] = fp8.dequantize(codes, sc[:, None])[:, None, :]
    hs = slice(hk * G, (hk + 1) * G)
    return oracle.decode_one(new["q"][b, hs], new["k"][b, hk:hk + 1], new["v"][b, hk:hk + 1], new["g"][b, hs],
                             hist["k"], hist["v"], lo, L_b, group_layer(lay))


@pytest.mark.parametrize("cfg", [wl.SPARK_DECODE_GLOBAL, wl.SPARK_DECODE_LOCAL], ids=lambda c: c.name + "_fp8")
def test_decode_fullsize_fp8_sampled(cfg):
    print(f"decode full size fp8 {cfg.name}", flush=True)
    y, lengths, extra = _decode_run(cfg, fp8=True)
    assert np.isfinite(y).all()
    new = sd.new_token_host(cfg)
    G = cfg.layer.group
    if cfg.layer.window:
        pairs = [(b, hk) for b in range(cfg.batch) for hk in range(cfg.layer.hkv)]
    else:
        pairs = paged_pairs(lengths, cfg.layer.hkv)
    worst = 0.0
    t = time.time()
    for b, hk in pairs:
        ref = oracle_decode_pair_fp8(cfg, new, b, hk, int(lengths[b]), extra)
        worst = max(worst, max_err(y[b, hk * G:(hk + 1) * G], ref))
    print(f"{cfg.name} fp8: {len(pairs)} pairs max_abs_err={worst:.3e} (oracle {time.time() - t:.1f} s)",
          flush=True)
    assert worst <= TOL


# 16 sequences of 20,000-30,000 positions over a paged cache: 8192-entry chunks
# would give only 256 * 5 workgroups, so the launch takes 4096-entry chunks (the
# full-size workload takes 8192, short test cases 2048).
MID_PAGED = dataclasses.replace(wl.SPARK_DECODE_GLOBAL, name="spark_decode_global_paged_mid", len_lo=20000,
                                len_hi=30000)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "e4m3"])
def test_decode_paged_middle_chunk_size(fp8):
    cfg = MID_PAGED
    print(f"decode {cfg.name} fp8={fp8}", flush=True)
    res = _decode_run(cfg, fp8=fp8)
    y, lengths = res[0], res[1]
    assert np.isfinite(y).all()
    new = sd.new_token_host(cfg)
    G = cfg.layer.group
    pairs = [(b, (5 * b) % cfg.layer.hkv) for b in range(cfg.batch)]
    worst = 0.0
    t = time.time()
    for b, hk in pairs:
        if fp8:
            ref = oracle_decode_pair_fp8(cfg, new, b, hk, int(lengths[b]), res[2])
        else:
            ref = oracle_decode_pair(cfg, new, b, hk, int(lengths[b]))
        worst = max(worst, max_err(y[b, hk * G:(hk + 1) * G], ref))
    print(f"{cfg.name}: {len(pairs)} pairs, lengths {int(lengths.min())}-{int(lengths.max())}, "
          f"max_abs_err={worst:.3e} (oracle {time.time() - t:.1f} s)", flush=True)
    assert worst <= TOL


# 48 sequences of the Spark global layer with lengths on and around multiples
# of 8192: the launch takes 8192-entry chunks (768 * 3 workgroups), so every
# chunk edge case of that size is checked, one KV head per sequence.
EDGE_LENGTHS = [1, 2, 31, 32, 33, 8191, 8192, 8193, 8194, 16383, 16384, 16385] * 4
EDGE_PAGED = dataclasses.replace(wl.SPARK_DECODE_GLOBAL, name="spark_decode_global_paged_chunk_edges", batch=48,
                                 len_lo=1, len_hi=16400)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "e4m3"])
def test_decode_paged_chunk_edges(fp8):
    cfg = EDGE_PAGED
    print(f"decode {cfg.name} fp8={fp8}", flush=True)
    res = _decode_run(cfg, fp8=fp8, lengths=EDGE_LENGTHS)
    y, lengths = res[0], res[1]
    assert list(lengths) == EDGE_LENGTHS
    assert np.isfinite(y).all()
    new = sd.new_token_host(cfg)
    G = cfg.layer.group
    worst = 0.0
    for b in range(cfg.batch):
        hk = (7 * b) % cfg.layer.hkv
        if fp8:
            ref = oracle_decode_pair_fp8(cfg, new, b, hk, int(lengths[b]), res[2])
        else:
            ref = oracle_decode_pair(cfg, new, b, hk, int(lengths[b]))
        worst = max(worst, max_err(y[b, hk * G:(hk + 1) * G], ref))
    print(f"{cfg.name}: {cfg.batch} sequences, max_abs_err={worst:.3e}", flush=True)
    assert worst <= TOL


@pytest.mark.parametrize("cfg", wl.CHUNK, ids=lambda c: c.name)
def test_prefill_chunk_fullsize_sampled(cfg):
    """A 2048-token chunk after 131072 cached positions: sampled rows of two
    KV-head groups against the oracle over the whole visible history, and
    the appended values in the cache."""
    L = cfg.layer
    G = L.group
    print(f"chunk full size {cfg.name}", flush=True)
    s = sd.chunk_device_setup(cfg)
    if s["kind"] == "ring":
        cache = ma.KvCache.ring(s["kc"], s["vc"])
    else:
        cache = ma.KvCache.paged(s["kc"], s["vc"], s["block_table"], s["page_tokens"])
    lp = ma.LayerParams.from_layer(L)
    y = ma.prefill_chunk(lp, s["q"], s["k"], s["v"], s["g"], s["start"], cfg.start, cache)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    y = y.float().cpu().numpy()
    S, T = cfg.start, cfg.seq
    rows = sample_rows(T, 0, n_random=6)
    worst = 0.0
    t = time.time()
    for hk in sorted({0, L.hkv - 1}):
        heads = np.arange(hk * G, (hk + 1) * G)
        hs = max(0, S - L.window + 1) if L.window else 0
        k_hist = sd.cache_values_host(cfg.seed, 0, hk, L.hkv, "k", hs, S, L.d)[:, None, :]
        v_hist = sd.cache_values_host(cfg.seed, 0, hk, L.hkv, "v", hs, S, L.d)[:, None, :]
        kc = sd.chunk_host_rows(cfg, "k", 0, np.arange(T), [hk])
        vch = sd.chunk_host_rows(cfg, "v", 0, np.arange(T), [hk])
        q = sd.chunk_host_rows(cfg, "q", 0, rows, heads)
        g = sd.chunk_host_rows(cfg, "g", 0, rows, heads)
        ref = oracle.prefill_chunk(q, kc, vch, g, k_hist, v_hist, hs, S, group_layer(L), rows=rows)
        worst = max(worst, max_err(y[0][rows][:, heads], ref))
        # the chunk's values were appended (exact copies)
        for r in rows:
            p = S + r
            if s["kind"] == "ring":
                if r < T - L.window:
                    continue
                got = s["vc"][0, hk, :, p % L.window]
            else:
                pt = s["page_tokens"]
                got = s["vc"][int(s["table_host"][0, p // pt]), hk, :, p % pt]
            assert np.array_equal(got.float().cpu().numpy(), vch[r, 0])
    print(f"{cfg.name}: {len(rows)} rows x {2 * G} heads, max_abs_err={worst:.3e} (oracle {time.time() - t:.1f} s)",
          flush=True)
    assert worst <= TOL


def test_draft_block_fullsize_sampled():
    """The drafter's 16-token block after 131072 cached positions (16
    sequences, a 2048-entry ring): every row of two KV-head groups of the
    first and last sequence against the oracle over the visible context, and
    the cache left bit-for-bit unchanged."""
    cfg = wl.GLIMMER_DRAFT_BLOCK
    L = cfg.layer
    G = L.group
    print(f"draft block full size {cfg.name}", flush=True)
    s = sd.chunk_device_setup(cfg)
    assert s["kind"] == "ring"
    cache = ma.KvCache.ring(s["kc"], s["vc"])
    k_before, v_before = s["kc"].clone(), s["vc"].clone()
    lp = ma.LayerParams.from_layer(L)
    ws = torch.empty(ma.draft_block_workspace_size(lp, cfg.batch, cfg.seq, cfg.start), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(s["q"])
    y = ma.draft_block(lp, s["q"], s["k"], s["v"], s["g"], s["start"], cfg.start, cache, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    assert torch.equal(s["kc"], k_before) and torch.equal(s["vc"], v_before)
    y = y.float().cpu().numpy()
    S, T = cfg.start, cfg.seq
    hs = S - L.window + 1                       # the first row's window starts here
    rows = np.arange(T)
    worst = 0.0
    t = time.time()
    for b in sorted({0, cfg.batch - 1}):
        for hk in sorted({0, L.hkv - 1}):
            heads = np.arange(hk * G, (hk + 1) * G)
            k_hist = sd.cache_values_host(cfg.seed, b, hk, L.hkv, "k", hs, S, L.d)[:, None, :]
            v_hist = sd.cache_values_host(cfg.seed, b, hk, L.hkv, "v", hs, S, L.d)[:, None, :]
            kb = sd.chunk_host_rows(cfg, "k", b, rows, [hk])
            vb = sd.chunk_host_rows(cfg, "v", b, rows, [hk])
            q = sd.chunk_host_rows(cfg, "q", b, rows, heads)
            g = sd.chunk_host_rows(cfg, "g", b, rows, heads)
            ref = oracle.block_bidirectional(q, kb, vb, g, k_hist, v_hist, hs, S, group_layer(L))
            worst = max(worst, max_err(y[b][:, heads], ref))
    print(f"{cfg.name}: 2 sequences x {2 * G} heads x {T} rows, max_abs_err={worst:.3e} "
          f"(oracle {time.time() - t:.1f} s)", flush=True)
    assert worst <= TOL


def test_attention_block_fullsize_sampled():
    """The attention half of a Spark decoder block on 4096 tokens (hidden
    8192, local layer): sampled rows against the fp64 block oracle.  A row
    of a local layer depends on the hidden states of its own window only, so
    the oracle runs on the slice of rows that ends at the sampled row and
    starts at its window's first position (or at 0)."""
    from oracle import block as OB
    from synth.device import block_device_setup
    from test_gpu_block import beyond_half_ulp
    cfg = wl.SPARK_BLOCK_LOCAL
    L = cfg.layer
    W = L.window
    assert W > 0 and cfg.batch == 1
    print(f"attention block full size {cfg.name}", flush=True)
    s = block_device_setup(cfg)
    w = ma.BlockWeights(in_norm=s["in_norm"], w_qkvg=s["w_qkvg"], w_o=s["w_o"], residual_gate=s["residual_gate"],
                        post_norm=s["post_norm"])
    lp = ma.LayerParams.from_layer(L)
    ws = torch.empty(ma.block_prefill_workspace_size(lp, w, cfg.batch, cfg.seq), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(s["x"])
    y = ma.attention_block_prefill(lp, w, s["x"], out=out, workspace=ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    y = y[0].float().cpu().numpy()

    def host(t):
        return t.double().cpu().numpy() if t is not None else None

    Wt = {"in_norm": host(s["in_norm"]), "w_qkvg": host(s["w_qkvg"]), "w_o": host(s["w_o"]),
          "post_norm": host(s["post_norm"]), "residual_gate": host(s["residual_gate"])}
    x = host(s["x"][0])
    T = cfg.seq
    # one slice from 0 covers every row whose window starts at 0; later rows
    # each get the slice of their own window
    early = [r for r in sample_rows(T, W, n_random=0) if r < W]
    late = sorted({T - 1, T - 2, W, W + 1, *np.random.default_rng(3).integers(W, T, size=2).tolist()})
    worst = 0.0
    t = time.time()
    ref = OB.attention_block(x[:W], Wt, L, rows=np.array(early))
    worst = max(worst, beyond_half_ulp(y[early], ref))
    for r in late:
        lo = r - W + 1
        ref = OB.attention_block(x[lo:r + 1], Wt, L, positions=np.arange(lo, r + 1), rows=np.array([W - 1]))
        worst = max(worst, beyond_half_ulp(y[[r]], ref))
    # the block tests' bar: TOL on the error beyond the output's own bf16 rounding
    print(f"{cfg.name}: {len(early) + len(late)} rows x {cfg.hidden}, max error beyond half an ulp={worst:.3e} "
          f"(oracle {time.time() - t:.1f} s)", flush=True)
    assert worst <= TOL
