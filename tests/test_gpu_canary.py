"""Canaries around every entry point's buffers, through the C ABI.

Each call runs twice on the same inputs: once with a zeroed workspace and
output, once with the workspace filled with NaN bytes (0xFF: a NaN as bf16,
fp16 and fp32) and the output pre-filled with a NaN of a marked payload.
The second run must give the first run's output bit for bit (no kernel may
read workspace or output bytes it has not written in the same call), every
output element finite, and the canaries must come back untouched: guard
bytes after the workspace's required size, and guard rows and heads around
the output (a strided view into a larger buffer where the call takes
strides, guard elements after it where it takes a contiguous tensor).  A
call that writes a cache does so identically in both runs."""
import numpy as np
import pytest
import torch

import global_muse_rope_amd as ma
import synth
from synth.workloads import Layer, GLIMMER_SCALE, SPARK_SCALE
from gpu_helpers import TOL, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"
GUARD_BYTE = 0xA5
GUARD_BF16 = 0x7FA5          # a quiet NaN with a payload no kernel writes
GUARD_BYTES = 4096


def _workspace(need, poison):
    """A need-byte workspace (zeros, or 0xFF) followed by GUARD_BYTES guard bytes."""
    buf = torch.full((need + GUARD_BYTES,), GUARD_BYTE, dtype=torch.uint8, device=DEV)
    buf[:need] = 0xFF if poison else 0
    return buf, buf[:need]


def _guard_intact(buf, need):
    return bool(torch.all(buf[need:] == GUARD_BYTE))


def _nan_bf16(shape):
    t = torch.full(shape, GUARD_BF16, dtype=torch.int16, device=DEV)
    return t.view(torch.bfloat16)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu()


def _strided_out(B, T, H, D, poison):
    """out [B, T, H, D] as a view into [B, T + 2, H + 2, D] whose border rows and heads are guards."""
    big = _nan_bf16((B, T + 2, H + 2, D))
    out = big[:, 1:T + 1, 1:H + 1]
    if not poison:
        out.zero_()
    return big, out


def _border_intact(big):
    g = big.view(torch.int16)
    return bool(torch.all(g[:, 0] == GUARD_BF16) and torch.all(g[:, -1] == GUARD_BF16)
                and torch.all(g[:, :, 0] == GUARD_BF16) and torch.all(g[:, :, -1] == GUARD_BF16))


def _flat_out(shape, poison):
    """out of `shape` (contiguous) followed by GUARD_BYTES / 2 guard elements."""
    n = int(np.prod(shape))
    big = _nan_bf16((n + GUARD_BYTES // 2,))
    out = big[:n].view(shape)
    if not poison:
        out.zero_()
    return big, out


def _tail_intact(big, n):
    return bool(torch.all(big.view(torch.int16)[n:] == GUARD_BF16))


def _check_pair(clean, canary, exact=True):
    assert torch.isfinite(canary.float()).all(), "non-finite output under a poisoned workspace"
    if exact:
        assert torch.equal(_bits(clean), _bits(canary)), "output depends on workspace or output contents"
    else:
        assert torch.allclose(clean.float(), canary.float(), rtol=0, atol=TOL)


def _inputs(layer, B, T, seed):
    shp = {"q": (B, T, layer.hq, layer.d), "k": (B, T, layer.hkv, layer.d),
           "v": (B, T, layer.hkv, layer.d), "g": (B, T, layer.hq, layer.d)}
    return {n: to_dev(synth.normal_bf16_bits(seed, i + 1, s)) for i, (n, s) in enumerate(shp.items())}


def _clone_cache(c):
    if c.block_table is None:
        return ma.KvCache.ring(c.k.clone(), c.v.clone(), c.k_scale, c.v_scale)
    return ma.KvCache.paged(c.k.clone(), c.v.clone(), c.block_table, c.page_tokens, c.k_scale, c.v_scale)


SPARK = dict(hq=16, hkv=2, d=64, scale=SPARK_SCALE, out_norm=True, out_eps=1e-6)
GLIMMER = dict(hq=32, hkv=2, d=128, scale=GLIMMER_SCALE)

PREFILL_CASES = [
    # (layer, B, T): several query blocks and key tiles, ragged tails; the short global
    # sequence splits its keys over workgroups (partials in the workspace)
    (Layer(window=256, theta=10000.0, **GLIMMER), 2, 700),
    (Layer(window=0, theta=0.0, **GLIMMER), 1, 333),
    (Layer(window=128, theta=10000.0, **SPARK), 2, 1001),
    (Layer(window=0, theta=0.0, **SPARK), 1, 1500),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: f"d{c[0].d}w{c[0].window}B{c[1]}T{c[2]}")
def test_prefill_canaries(case):
    layer, B, T = case
    lp = ma.LayerParams.from_layer(layer)
    x = _inputs(layer, B, T, 21)
    need = ma.prefill_workspace_size(lp, B, T)
    outs = []
    for poison in (False, True):
        buf, ws = _workspace(need, poison)
        big, out = _strided_out(B, T, layer.hq, layer.d, poison)
        print(f"prefill canary {layer} B={B} T={T} poison={poison}", flush=True)
        ma.prefill(lp, x["q"], x["k"], x["v"], x["g"], out=out, workspace=ws)
        torch.cuda.synchronize()
        assert _guard_intact(buf, need), "write past the workspace's required size"
        assert _border_intact(big), "write outside the output view"
        outs.append(out)
    _check_pair(*outs)


def _chunk_cache(kind, layer, starts, T, pt):
    from test_gpu_chunk import make_chunk_cache
    return make_chunk_cache(kind, layer, starts, T, pt, False)[0]


CHUNK_CASES = [
    # (entry, kind, layer, starts, T, page_tokens)
    ("chunk", "ring", Layer(window=256, theta=10000.0, **SPARK), [0, 40, 700], 300, 32),
    ("chunk", "paged", Layer(window=0, theta=0.0, **GLIMMER), [0, 77, 300], 130, 16),
    ("chunk", "paged", Layer(window=0, theta=0.0, **SPARK), [5, 1000], 40, 32),   # few blocks: key split
    ("draft", "ring", Layer(hq=32, hkv=8, d=128, window=2048, theta=10000.0, scale=GLIMMER_SCALE),
     [0, 5, 2047, 3000], 16, 32),                                                    # few-token split path
    ("draft", "paged", Layer(window=0, theta=0.0, **SPARK), [0, 63, 300], 150, 16),  # tile path
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: f"{c[0]}-{c[1]}-d{c[2].d}w{c[2].window}T{c[4]}")
def test_chunk_and_draft_canaries(case):
    entry, kind, layer, starts, T, pt = case
    B = len(starts)
    lp = ma.LayerParams.from_layer(layer)
    x = _inputs(layer, B, T, 22)
    base = _chunk_cache(kind, layer, starts, T, pt)
    st = torch.tensor(starts, dtype=torch.int32, device=DEV)
    ms = int(max(starts))
    fn = ma.prefill_chunk if entry == "chunk" else ma.draft_block
    size = ma.prefill_chunk_workspace_size if entry == "chunk" else ma.draft_block_workspace_size
    need = size(lp, B, T, ms)
    outs, caches = [], []
    for poison in (False, True):
        cache = _clone_cache(base)
        buf, ws = _workspace(need, poison)
        big, out = _strided_out(B, T, layer.hq, layer.d, poison)
        print(f"{entry} canary {kind} {layer} starts={starts} T={T} poison={poison}", flush=True)
        fn(lp, x["q"], x["k"], x["v"], x["g"], st, ms, cache, out=out, workspace=ws)
        torch.cuda.synchronize()
        assert _guard_intact(buf, need), "write past the workspace's required size"
        assert _border_intact(big), "write outside the output view"
        outs.append(out)
        caches.append(cache)
    _check_pair(*outs)
    assert torch.equal(caches[0].k, caches[1].k) and torch.equal(caches[0].v, caches[1].v)


DECODE_CASES = [
    # (kind, layer, kv lengths, page_tokens)
    ("paged", Layer(window=0, theta=0.0, **SPARK), [300, 77, 1, 2, 33, 64], 32),
    ("paged", Layer(window=0, theta=0.0, **GLIMMER), [5000, 4097, 4096, 17], 16),
    ("ring", Layer(window=256, theta=10000.0, **SPARK), [1, 2, 255, 256, 257, 1000], 0),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"{c[0]}-d{c[1].d}w{c[1].window}")
def test_decode_canaries(case):
    from test_gpu_parity import make_cache
    kind, layer, lens, pt = case
    B = len(lens)
    lens = np.array(lens, dtype=np.int32)
    base, _, _ = make_cache(kind, layer, B, lens, page_tokens=pt or 32)
    lp = ma.LayerParams.from_layer(layer)
    new = {n: to_dev(synth.normal_bf16_bits(23, i + 1, s)) for i, (n, s) in enumerate(
        [("q", (B, layer.hq, layer.d)), ("k", (B, layer.hkv, layer.d)), ("v", (B, layer.hkv, layer.d)),
         ("g", (B, layer.hq, layer.d))])}
    kv = torch.from_numpy(lens).to(DEV)
    need = ma.decode_workspace_size(lp, B, int(lens.max()), base)
    n = B * layer.hq * layer.d
    outs, caches = [], []
    for poison in (False, True):
        cache = _clone_cache(base)
        buf, ws = _workspace(need, poison)
        big, out = _flat_out((B, layer.hq, layer.d), poison)
        print(f"decode canary {kind} {layer} lens={lens.tolist()} poison={poison}", flush=True)
        ma.decode(lp, new["q"], new["k"], new["v"], new["g"], kv, int(lens.max()), cache, out=out, workspace=ws)
        torch.cuda.synchronize()
        assert _guard_intact(buf, need), "write past the workspace's required size"
        assert _tail_intact(big, n), "write past the output"
        outs.append(out)
        caches.append(cache)
    _check_pair(*outs)
    assert torch.equal(caches[0].k, caches[1].k) and torch.equal(caches[0].v, caches[1].v)


def test_block_canaries():
    """The decoder block's prefill and decode: its workspace holds the
    projections, the GEMM scratch and the layer's own workspace.  The
    projection GEMMs come from hipBLASLt, whose summation order is its own
    business, so the two runs agree within the layer's tolerance."""
    from test_gpu_block import make_block
    from test_gpu_parity import make_cache
    layer = Layer(hq=16, hkv=2, d=64, window=128, theta=10000.0, scale=SPARK_SCALE, out_norm=True, out_eps=1e-6)
    hidden, B, T = 768, 2, 200
    _, wb = make_block(layer, hidden, True)
    lp = ma.LayerParams.from_layer(layer)
    x = to_dev(synth.normal_bf16_bits(24, 9, (B, T, hidden)))
    need = ma.block_prefill_workspace_size(lp, wb, B, T)
    outs = []
    for poison in (False, True):
        buf, ws = _workspace(need, poison)
        big, out = _flat_out((B, T, hidden), poison)
        print(f"block prefill canary poison={poison}", flush=True)
        ma.attention_block_prefill(lp, wb, x, out=out, workspace=ws)
        torch.cuda.synchronize()
        assert _guard_intact(buf, need) and _tail_intact(big, B * T * hidden)
        outs.append(out)
    _check_pair(*outs, exact=False)

    lens = np.array([1, 2, 255, 256, 1000], dtype=np.int32)
    Bd = len(lens)
    base, _, _ = make_cache("ring", Layer(hq=16, hkv=2, d=64, window=256, theta=10000.0, scale=SPARK_SCALE,
                                          out_norm=True, out_eps=1e-6), Bd, lens)
    dl = ma.LayerParams.from_layer(Layer(hq=16, hkv=2, d=64, window=256, theta=10000.0, scale=SPARK_SCALE,
                                         out_norm=True, out_eps=1e-6))
    xd = to_dev(synth.normal_bf16_bits(25, 9, (Bd, hidden)))
    kv = torch.from_numpy(lens).to(DEV)
    need = ma.block_decode_workspace_size(dl, wb, Bd, int(lens.max()), base)
    outs = []
    for poison in (False, True):
        cache = _clone_cache(base)
        buf, ws = _workspace(need, poison)
        big, out = _flat_out((Bd, hidden), poison)
        print(f"block decode canary poison={poison}", flush=True)
        ma.attention_block_decode(dl, wb, xd, kv, int(lens.max()), cache, out=out, workspace=ws)
        torch.cuda.synchronize()
        assert _guard_intact(buf, need) and _tail_intact(big, Bd * hidden)
        outs.append(out)
    _check_pair(*outs, exact=False)
