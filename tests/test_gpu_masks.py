"""Exact mask and index checks of chunked prefill and of the drafter's
non-causal block, through the C ABI.

q = 0 makes every visible logit exactly 0, so each visible key gets weight
exactly 1/count.  V is one-hot by position: output dim c marks position
m0 + c, for the cached history (cache V) and the chunk's own tokens (the v
input) alike.  Output dim c of a row is nonzero iff position m0 + c is
visible to that row, so the visible set of every row is read off bit for
bit and compared with the oracle's visible_range (causal chunk) or
bidirectional_range (drafter block).  Every cache entry the call may not rely
on (positions outside the window the header requires, a ring's stale slot,
pages past the chunk start) holds NaN: reading one as a visible entry, or
meeting one with a zero weight, would show up in the output.  The workspace
is filled with NaN bytes before each call for the same reason."""
import numpy as np
import pytest
import torch

import global_muse_rope_amd as ma
import oracle
import synth
from synth.workloads import Layer

pytestmark = pytest.mark.gpu
DEV = "cuda"

BF16_ONE, BF16_NAN = 0x3F80, 0x7FC0
E4M3_ONE, E4M3_NAN = 0x38, 0x7F


def _dev_bits(a, fp8):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t if fp8 else t.view(torch.int16).view(torch.bfloat16)).to(DEV)


def _cache_positions(starts, W):
    """Positions each sequence's cache must hold: the visible history below its start."""
    return [np.arange(max(0, s - W + 1) if W else 0, s) for s in starts]


def _build(kind, layer, starts, T, pt, fp8, m0, table, n_pages):
    """Cache and chunk values for one marker window m0 .. m0 + D - 1."""
    d, hkv, W = layer.d, layer.hkv, layer.window
    B = len(starts)
    one, nan = (E4M3_ONE, E4M3_NAN) if fp8 else (BF16_ONE, BF16_NAN)
    dt = np.uint8 if fp8 else np.uint16
    if kind == "ring":
        kc = np.full((B, hkv, W, d), nan, dtype=dt)
        vc = np.full((B, hkv, d, W), nan, dtype=dt)
    else:
        kc = np.full((n_pages, hkv, pt, d), nan, dtype=dt)
        vc = np.full((n_pages, hkv, d, pt), nan, dtype=dt)
    for b, ps in enumerate(_cache_positions(starts, W)):
        for p in ps:
            if kind == "ring":
                kc[b, :, p % W, :] = 0
                vc[b, :, :, p % W] = 0
                if 0 <= p - m0 < d:
                    vc[b, :, p - m0, p % W] = one
            else:
                pg, r = table[b, p // pt], p % pt
                kc[pg, :, r, :] = 0
                vc[pg, :, :, r] = 0
                if 0 <= p - m0 < d:
                    vc[pg, :, p - m0, r] = one
    v = np.zeros((B, T, hkv, d), dtype=np.uint16)
    for b, s in enumerate(starts):
        for t in range(T):
            if 0 <= s + t - m0 < d:
                v[b, t, :, s + t - m0] = BF16_ONE
    return kc, vc, v


def run_marker_case(kind, layer, starts, T, draft, pt=32, fp8=False):
    d, hkv, hq, W = layer.d, layer.hkv, layer.hq, layer.window
    B = len(starts)
    max_start = int(max(starts))
    lp = ma.LayerParams.from_layer(layer)
    pages = (max_start + T + pt - 1) // pt
    n_pages = B * pages + 2
    table = np.random.default_rng(5).permutation(n_pages)[:B * pages].astype(np.int32).reshape(B, pages)
    table_dev = torch.from_numpy(table).to(DEV)
    n_scale = B * hkv if kind == "ring" else n_pages * hkv
    ks = torch.ones(n_scale, dtype=torch.float32, device=DEV)
    vs = torch.full((n_scale,), 0.5, dtype=torch.float32, device=DEV)
    q = torch.zeros((B, T, hq, d), dtype=torch.bfloat16, device=DEV)
    g = torch.full((B, T, hq, d), 30.0, dtype=torch.bfloat16, device=DEV)
    k = torch.from_numpy(synth.normal_bf16_bits(11, 2, (B, T, hkv, d)).view(np.int16)).view(torch.bfloat16).to(DEV)
    st = torch.tensor(starts, dtype=torch.int32, device=DEV)
    # the visible range of every (sequence, chunk row), absolute positions
    lo = np.zeros((B, T), dtype=np.int64)
    hi = np.zeros((B, T), dtype=np.int64)
    for b, s in enumerate(starts):
        for t in range(T):
            if draft:
                lo[b, t], hi[b, t] = oracle.bidirectional_range(s + t, W, s + T - 1)
            else:
                lo[b, t], hi[b, t] = oracle.visible_range(s + t, W)
    fn = ma.draft_block if draft else ma.prefill_chunk
    size_fn = ma.draft_block_workspace_size if draft else ma.prefill_chunk_workspace_size
    # the workspace holds NaN bytes: a read of anything the call did not write there shows up too
    ws = torch.full((max(size_fn(lp, B, T, max_start), 1),), 0xFF, dtype=torch.uint8, device=DEV)
    for m0 in range(0, max_start + T, d):
        kc, vc, v = _build(kind, layer, starts, T, pt, fp8, m0, table, n_pages)
        kcd, vcd = _dev_bits(kc, fp8), _dev_bits(vc, fp8)
        if kind == "ring":
            cache = ma.KvCache.ring(kcd, vcd, ks.view(B, hkv) if fp8 else None, vs.view(B, hkv) if fp8 else None)
        else:
            cache = ma.KvCache.paged(kcd, vcd, table_dev, pt, ks.view(n_pages, hkv) if fp8 else None,
                                     vs.view(n_pages, hkv) if fp8 else None)
        vd = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(DEV)
        ws.fill_(0xFF)
        y = fn(lp, q, k, vd, g, st, max_start, cache, workspace=ws)
        torch.cuda.synchronize()
        yf = y.float().cpu().numpy()                                 # [B, T, Hq, D]
        assert np.all(np.isfinite(yf)), f"non-finite output, markers from {m0}"
        m = m0 + np.arange(d)
        expect = (m[None, None, :] >= lo[:, :, None]) & (m[None, None, :] <= hi[:, :, None])   # [B, T, D]
        seen = yf != 0
        for h in range(hq):
            bad = np.argwhere(seen[:, :, h, :] != expect)
            assert bad.size == 0, (f"{'block' if draft else 'chunk'} {kind} W={W} head {h} markers from {m0}: "
                                   f"(b, t, c) {bad[:5].tolist()}")


def _lay(d, w, g=4):
    hkv = 2
    return Layer(hq=g * hkv, hkv=hkv, d=d, window=w, theta=10000.0 if w else 0.0, scale=1.0)


CHUNK_CASES = [
    # (kind, layer, starts, T, page_tokens)
    ("ring", _lay(64, 64), [0, 1, 63, 64, 65, 127, 128, 129, 200], 100, 0),            # T > W
    ("ring", _lay(64, 256, g=8), [0, 63, 64, 255, 256, 257, 511, 512, 700], 70, 0),
    ("ring", _lay(128, 2048, g=16), [0, 63, 2047, 2048, 2049, 4095, 4096], 64, 0),
    ("paged", _lay(64, 0), [0, 1, 63, 64, 65, 500, 1023], 90, 32),
    ("paged", _lay(64, 256), [0, 255, 256, 257, 300], 50, 32),                      # a local layer over pages
    ("paged", _lay(128, 0, g=16), [0, 17, 128, 640], 130, 16),
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: f"{c[0]}-d{c[1].d}w{c[1].window}T{c[3]}")
def test_chunk_visibility_exact(case):
    kind, layer, starts, T, pt = case
    run_marker_case(kind, layer, starts, T, draft=False, pt=pt or 32)


BLOCK_CASES = [
    ("ring", _lay(64, 64), [0, 1, 63, 64, 65, 128, 200], 150, 0),                     # block wider than W
    ("ring", _lay(64, 256, g=8), [0, 255, 256, 257, 512, 600], 16, 0),
    ("ring", _lay(128, 2048, g=16), [0, 2047, 2048, 2049, 4096], 16, 0),
    ("paged", _lay(64, 0), [0, 1, 64, 65, 300], 16, 32),
    ("paged", _lay(64, 0, g=8), [0, 63, 130], 150, 16),                               # block wider than a tile
    ("paged", _lay(64, 256), [0, 256, 257, 400], 40, 32),
    # blocks of at most 64 tokens and 128 (token, head) columns per KV head: the few-token decode path
    ("ring", _lay(128, 2048, g=4), [0, 2047, 2048, 2049, 4096], 16, 0),
    ("paged", _lay(64, 256), [0, 31, 256, 257, 400], 32, 32),
    ("paged", _lay(128, 0, g=2), [0, 17, 128, 640, 3000], 64, 16),
    ("ring", _lay(64, 64, g=8), [0, 1, 63, 64, 65, 200], 3, 0),
]


@pytest.mark.parametrize("case", BLOCK_CASES, ids=lambda c: f"{c[0]}-d{c[1].d}w{c[1].window}T{c[3]}")
def test_draft_block_visibility_exact(case):
    kind, layer, starts, T, pt = case
    run_marker_case(kind, layer, starts, T, draft=True, pt=pt or 32)


@pytest.mark.parametrize("draft", [False, True], ids=["chunk", "block"])
@pytest.mark.parametrize("kind", ["ring", "paged"])
def test_visibility_exact_e4m3(kind, draft):
    """The same over E4M3 caches: marker code 1.0 times a value scale of 0.5,
    NaN codes in every entry the call may not rely on."""
    layer = _lay(64, 256)
    run_marker_case(kind, layer, [0, 255, 256, 300], 40, draft=draft, pt=32, fp8=True)


@pytest.mark.parametrize("kind", ["ring", "paged"])
def test_draft_few_token_visibility_exact_e4m3(kind):
    """E4M3 caches on the drafter's few-token path (24 tokens x 4 heads per KV head)."""
    run_marker_case(kind, _lay(64, 256), [0, 255, 256, 300], 24, draft=True, pt=32, fp8=True)
