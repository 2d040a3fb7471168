"""Workload inputs generated directly in device memory (same bits as the host
forms in ``synth``), and host regeneration of any slice for the oracle.

Prefill tensors are indexed in the canonical layout [B, T, H, D].  Decode:
the new token's q, k, v, gate are [B, H, D]; cached entries of (sequence b,
KV head h) at position p are element p * D + d of stream
S_CACHE_BASE + 2 * (b * Hkv + h) (+1 for values).  A cache holds keys
after the layer's norm (and RoPE on local layers), so every cached key row
has mean square 1: cached keys are drawn as random signs, +1 or -1 per
element, which gives exactly that with no arithmetic of the layer here (a
rotation keeps the mean square, and a random direction stays random).
Cached values are N(0,1), like raw projections.  Paged caches place each sequence's pages at positions drawn from a
seeded permutation of the pool.

FP8 caches hold E4M3 codes drawn directly from the same streams (magnitude
codes 0x20 .. 0x47 with a random sign, no rounding of any value) and seeded
float32 scales in [0.3, 0.6) per (page, head) or per (sequence, head).
"""
from __future__ import annotations

import numpy as np

from . import (normal_bf16_torch, normal_bf16_torch_tensor, bf16_bits_to_f64, f32_to_bf16_bits, normal_f32,
               e4m3_codes, e4m3_codes_torch, sign_bf16_torch)
from .workloads import (S_Q, S_K, S_V, S_G, S_CACHE_BASE, S_X, S_IN_NORM, S_W_QKVG, S_W_O, S_POST_NORM, S_RES_GATE,
                        decode_lengths)

STREAM = {"q": S_Q, "k": S_K, "v": S_V, "g": S_G}


def prefill_shapes(cfg):
    L = cfg.layer
    return {"q": (cfg.batch, cfg.seq, L.hq, L.d), "k": (cfg.batch, cfg.seq, L.hkv, L.d),
            "v": (cfg.batch, cfg.seq, L.hkv, L.d), "g": (cfg.batch, cfg.seq, L.hq, L.d)}


def prefill_device_inputs(cfg, device="cuda"):
    return {n: normal_bf16_torch_tensor(cfg.seed, STREAM[n], shp, device)
            for n, shp in prefill_shapes(cfg).items()}


def host_rows(cfg, name, b, rows, heads=None):
    """float64 values of tensor `name` at batch b, token rows, given heads."""
    B, T, H, D = prefill_shapes(cfg)[name]
    rows = np.asarray(rows, dtype=np.int64)
    heads = np.arange(H) if heads is None else np.asarray(heads, dtype=np.int64)
    idx = ((b * T + rows[:, None, None]) * H + heads[None, :, None]) * D + np.arange(D)[None, None, :]
    return bf16_bits_to_f64(f32_to_bf16_bits(normal_f32(cfg.seed, STREAM[name], idx)))


def host_tokens(cfg, name, b, t0, t1, heads=None):
    """float64 values of tokens t0 .. t1-1 (all of `heads`) via the torch CPU form."""
    import torch
    B, T, H, D = prefill_shapes(cfg)[name]
    heads = np.arange(H) if heads is None else np.asarray(heads, dtype=np.int64)
    out = np.empty((t1 - t0, len(heads), D), dtype=np.float64)
    step = 1 << 15
    hh = torch.from_numpy(heads)[None, :, None]
    dd = torch.arange(D, dtype=torch.int64)[None, None, :]
    for s in range(t0, t1, step):
        e = min(t1, s + step)
        tok = torch.arange(s, e, dtype=torch.int64)[:, None, None]
        idx = ((b * T + tok) * H + hh) * D + dd
        out[s - t0:e - t0] = normal_bf16_torch(cfg.seed, STREAM[name], idx.reshape(-1)).float().numpy().reshape(
            e - s, len(heads), D)
    return out


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def cache_stream(b, h, hkv, which):
    return S_CACHE_BASE + 2 * (b * hkv + h) + (1 if which == "v" else 0)


def cache_values_torch(seed, b, h, hkv, which, p0, p1, d, device):
    """bf16 tensor [p1 - p0, d] of cached entries at positions p0 .. p1-1:
    keys are signs (unit mean square per row), values N(0,1)."""
    import torch
    idx = torch.arange(p0 * d, p1 * d, dtype=torch.int64, device=device)
    draw = sign_bf16_torch if which == "k" else normal_bf16_torch
    return draw(seed, cache_stream(b, h, hkv, which), idx).view(p1 - p0, d)


def cache_values_host(seed, b, h, hkv, which, p0, p1, d):
    """float64 [p1 - p0, d], the same values on the host."""
    vals = np.empty((p1 - p0, d), dtype=np.float64)
    step = 1 << 16
    for s in range(p0, p1, step):
        e = min(p1, s + step)
        vals[s - p0:e - p0] = cache_values_torch(seed, b, h, hkv, which, s, e, d, "cpu").float().numpy()
    return vals


def cache_codes_torch(seed, b, h, hkv, which, p0, p1, d, device):
    """uint8 E4M3 codes [p1 - p0, d] of cached entries at positions p0 .. p1-1."""
    import torch
    idx = torch.arange(p0 * d, p1 * d, dtype=torch.int64, device=device)
    return e4m3_codes_torch(seed, cache_stream(b, h, hkv, which), idx).view(p1 - p0, d)


def cache_codes_host(seed, b, h, hkv, which, p0, p1, d):
    """The same codes on the host (numpy uint8 [p1 - p0, d])."""
    idx = np.arange(p0 * d, p1 * d, dtype=np.int64)
    return e4m3_codes(seed, cache_stream(b, h, hkv, which), idx).reshape(p1 - p0, d)


def cache_scales(seed, shape):
    """Seeded float32 scales (k, v) in [0.3, 0.6) of the given shape."""
    rng = np.random.default_rng(seed + 3)
    return (rng.uniform(0.3, 0.6, shape).astype(np.float32), rng.uniform(0.3, 0.6, shape).astype(np.float32))


def new_token_shapes(cfg):
    L = cfg.layer
    return {"q": (cfg.batch, L.hq, L.d), "k": (cfg.batch, L.hkv, L.d), "v": (cfg.batch, L.hkv, L.d),
            "g": (cfg.batch, L.hq, L.d)}


def new_token_host(cfg):
    out = {}
    for n, shp in new_token_shapes(cfg).items():
        idx = np.arange(int(np.prod(shp)), dtype=np.int64)
        out[n] = bf16_bits_to_f64(f32_to_bf16_bits(normal_f32(cfg.seed + 1, STREAM[n], idx))).reshape(shp)
    return out


def decode_device_setup(cfg, device="cuda", lengths=None, fp8=False, plain_fill=False):
    """Ring (window > 0) or paged (global) cache filled for every sequence's
    history, the new-token tensors and kv_len.  Returns a dict of tensors:
    q, k, v, g, kv_len (int32), lengths (numpy), max_len, and the cache
    pieces kind, kc, vc, block_table, page_tokens; with ``fp8`` the pools
    hold E4M3 codes and the dict adds k_scale, v_scale (device) and
    scales_host (numpy k, v) and table_host (paged).  ``plain_fill`` fills
    each pool with one call of torch's own generator instead of the seeded
    per-sequence streams: the same shapes, lengths and page table, for runs
    whose figures do not depend on the cached values (byte counters)."""
    import torch
    L = cfg.layer
    d, hkv, B = L.d, L.hkv, cfg.batch
    lengths = decode_lengths(cfg.seed, B, cfg.len_lo, cfg.len_hi) if lengths is None else np.asarray(lengths)
    max_len = int(cfg.len_hi)
    res = {n: normal_bf16_torch_tensor(cfg.seed + 1, STREAM[n], shp, device)
           for n, shp in new_token_shapes(cfg).items()}
    res["kv_len"] = torch.from_numpy(lengths.astype(np.int32)).to(device)
    res["lengths"] = lengths
    res["max_len"] = max_len
    edt = torch.uint8 if fp8 else torch.bfloat16

    def plain(t):
        if fp8:
            return t.random_(0, 0x78)   # finite positive E4M3 codes
        return t.normal_()

    def values(b, h, which, p0, p1):
        if fp8:
            return cache_codes_torch(cfg.seed, b, h, hkv, which, p0, p1, d, device)
        return cache_values_torch(cfg.seed, b, h, hkv, which, p0, p1, d, device)

    def put_scales(shape):
        if fp8:
            ks, vs = cache_scales(cfg.seed, shape)
            res.update(k_scale=torch.from_numpy(ks).to(device), v_scale=torch.from_numpy(vs).to(device),
                       scales_host=(ks, vs))

    if L.window > 0:
        W = L.window
        kc = torch.zeros((B, hkv, W, d), dtype=edt, device=device)
        vc = torch.zeros((B, hkv, d, W), dtype=edt, device=device)
        if plain_fill:
            plain(kc)
            plain(vc)
        for b in range(B if not plain_fill else 0):
            n = int(lengths[b])
            p0, p1 = max(0, n - 1 - W), n - 1
            if p1 <= p0:
                continue
            slots = torch.arange(p0, p1, device=device) % W
            for h in range(hkv):
                kc[b, h, slots, :] = values(b, h, "k", p0, p1)
                vc[b, h, :, slots] = values(b, h, "v", p0, p1).t()
        res.update(kind="ring", kc=kc, vc=vc, block_table=None, page_tokens=0)
        put_scales((B, hkv))
        return res
    pt = cfg.page_tokens
    pages = [(int(n) + pt - 1) // pt for n in lengths]
    max_pages = (max_len + pt - 1) // pt
    n_pool = sum(pages) + 1
    perm = np.random.default_rng(cfg.seed + 2).permutation(n_pool).astype(np.int32)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]
    kc = torch.empty((n_pool, hkv, pt, d), dtype=edt, device=device)
    vc = torch.empty((n_pool, hkv, d, pt), dtype=edt, device=device)
    tdev = torch.from_numpy(table).to(device)
    if plain_fill:
        plain(kc)
        plain(vc)
    for b in range(B if not plain_fill else 0):
        n = int(lengths[b])
        idxp = tdev[b, :pages[b]].long()
        for h in range(hkv):
            for which, dst in (("k", kc), ("v", vc)):
                vals = torch.zeros((pages[b] * pt, d), dtype=edt, device=device)
                vals[:n] = values(b, h, which, 0, n)
                vals = vals.view(pages[b], pt, d)
                if which == "k":
                    dst[idxp, h] = vals
                else:
                    dst[idxp, h] = vals.transpose(1, 2)
    res.update(kind="paged", kc=kc, vc=vc, block_table=tdev, page_tokens=pt, table_host=table)
    put_scales((n_pool, hkv))
    return res


# ---------------------------------------------------------------------------
# chunked prefill
# ---------------------------------------------------------------------------

def chunk_device_setup(cfg, device="cuda"):
    """A chunk workload: the chunk's q, k, v, g [B, T, H, D] (prefill streams,
    seed + 5) and a cache holding positions 0 .. start - 1 of every sequence
    (cache streams, the decode recipe): a ring (local layer) keeps the last W,
    a paged cache maps pages for start + T positions from a seeded
    permutation.  Returns a dict of tensors plus kind, page_tokens and (paged)
    table_host."""
    import torch
    L = cfg.layer
    d, hkv, B, T, S = L.d, L.hkv, cfg.batch, cfg.seq, cfg.start
    res = {n: normal_bf16_torch_tensor(cfg.seed + 5, STREAM[n], shp, device)
           for n, shp in [("q", (B, T, L.hq, d)), ("k", (B, T, hkv, d)), ("v", (B, T, hkv, d)),
                          ("g", (B, T, L.hq, d))]}
    res["start"] = torch.full((B,), S, dtype=torch.int32, device=device)
    if L.window > 0:
        W = L.window
        kc = torch.zeros((B, hkv, W, d), dtype=torch.bfloat16, device=device)
        vc = torch.zeros((B, hkv, d, W), dtype=torch.bfloat16, device=device)
        p0 = max(0, S - W)
        slots = torch.arange(p0, S, device=device) % W
        for b in range(B):
            for h in range(hkv):
                kc[b, h, slots, :] = cache_values_torch(cfg.seed, b, h, hkv, "k", p0, S, d, device)
                vc[b, h, :, slots] = cache_values_torch(cfg.seed, b, h, hkv, "v", p0, S, d, device).t()
        res.update(kind="ring", kc=kc, vc=vc, block_table=None, page_tokens=0)
        return res
    pt = cfg.page_tokens
    pages = (S + T + pt - 1) // pt
    n_pool = B * pages
    table = np.random.default_rng(cfg.seed + 2).permutation(n_pool).astype(np.int32).reshape(B, pages)
    kc = torch.zeros((n_pool, hkv, pt, d), dtype=torch.bfloat16, device=device)
    vc = torch.zeros((n_pool, hkv, d, pt), dtype=torch.bfloat16, device=device)
    tdev = torch.from_numpy(table).to(device)
    hp = (S + pt - 1) // pt
    for b in range(B):
        idxp = tdev[b, :hp].long()
        for h in range(hkv):
            for which, dst in (("k", kc), ("v", vc)):
                vals = torch.zeros((hp * pt, d), dtype=torch.bfloat16, device=device)
                vals[:S] = cache_values_torch(cfg.seed, b, h, hkv, which, 0, S, d, device)
                vals = vals.view(hp, pt, d)
                dst[idxp, h] = vals if which == "k" else vals.transpose(1, 2)
    res.update(kind="paged", kc=kc, vc=vc, block_table=tdev, page_tokens=pt, table_host=table)
    return res


def chunk_host_rows(cfg, name, b, rows, heads=None):
    """float64 values of the chunk tensor `name` (q, k, v or g) at sequence
    b, chunk rows `rows`, heads `heads`."""
    L = cfg.layer
    H = L.hq if name in ("q", "g") else L.hkv
    rows = np.asarray(rows, dtype=np.int64)
    heads = np.arange(H) if heads is None else np.asarray(heads, dtype=np.int64)
    idx = (((b * cfg.seq + rows[:, None, None]) * H + heads[None, :, None]) * L.d
           + np.arange(L.d)[None, None, :])
    return bf16_bits_to_f64(f32_to_bf16_bits(normal_f32(cfg.seed + 5, STREAM[name], idx)))



def block_device_setup(cfg, device="cuda"):
    """Inputs of the decoder-block workload: hidden states x [B, T, hidden]
    (N(0,1) bf16) and seeded weights, each an N(0,1) bf16 draw times a fixed
    scale (an fp32 product rounded to bf16, nearest-even; the same bits on
    any device): input and post-attention norm weights 0.1, the stacked
    q/k/v/gate projection hidden^-1/2, o_proj (Hq D)^-1/2, and the fp32
    residual-gate parameter 0.5.  Returns a dict of tensors; exactly one of
    post_norm (Glimmer) and residual_gate (Spark) is set."""
    import torch
    L = cfg.layer
    H = cfg.hidden
    n = (2 * L.hq + 2 * L.hkv) * L.d

    def scaled(stream, shape, scale, dtype=torch.bfloat16):
        return (normal_bf16_torch_tensor(cfg.seed, stream, shape, device).float() * scale).to(dtype)

    res = {"x": normal_bf16_torch_tensor(cfg.seed, S_X, (cfg.batch, cfg.seq, H), device),
           "in_norm": scaled(S_IN_NORM, (H,), 0.1),
           "w_qkvg": scaled(S_W_QKVG, (n, H), H ** -0.5),
           "w_o": scaled(S_W_O, (H, L.hq * L.d), (L.hq * L.d) ** -0.5),
           "post_norm": None, "residual_gate": None}
    if cfg.spark:
        res["residual_gate"] = scaled(S_RES_GATE, (H,), 0.5, torch.float32)
    else:
        res["post_norm"] = scaled(S_POST_NORM, (H,), 0.1)
    return res
