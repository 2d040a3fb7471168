"""Work and byte accounting for the attention layer (host-side, no GPU).

The conventions are the pages': attention FLOPs count only the two
contractions, 4 * Hq * D per visible (query, key) pair per layer (Muse Spark
Open deep dive, section 7.3, the A(c) equation), and a cached token costs
2 * Hkv * D * 2 bytes per layer in bf16 (same page, section 1.2 table and the
KV(c) equation of section 7.2).
"""
from __future__ import annotations


def visible_pairs(seq: int, window: int) -> int:
    """Number of (query, key) pairs with key visible, over a causal sequence.

    Query i sees min(i + 1, W) keys on a local layer and i + 1 on a global
    one (window 0)."""
    if seq <= 0:
        return 0
    if window == 0 or window >= seq:
        return seq * (seq + 1) // 2
    return window * (window + 1) // 2 + (seq - window) * window


def flops_per_pair(hq: int, d: int) -> int:
    return 4 * hq * d


def prefill_flops(hq: int, d: int, batch: int, seq: int, window: int) -> int:
    return flops_per_pair(hq, d) * batch * visible_pairs(seq, window)


def block_pairs(start: int, seq: int, window: int) -> int:
    """Visible pairs of a non-causal block of `seq` tokens at positions start
    .. start + seq - 1: row t sees back to start + t - W + 1 (or position 0)
    and forward to the block's last position."""
    if window == 0:
        return seq * (start + seq)
    return sum(start + seq - max(0, start + t - window + 1) for t in range(seq))


def chunk_pairs(start: int, seq: int, window: int) -> int:
    """Visible (query, key) pairs of a chunk of `seq` tokens at positions
    start .. start + seq - 1: the tail of the whole sequence's pairs."""
    return visible_pairs(start + seq, window) - visible_pairs(start, window)


def kv_bytes_per_token(hkv: int, d: int, elem_bytes: int = 2) -> int:
    return 2 * hkv * d * elem_bytes


def draft_bytes(hq: int, hkv: int, d: int, batch: int, seq: int, start: int, window: int,
                elem_bytes: int = 2) -> int:
    """HBM bytes a drafter's block moves once: the cached K and V of the
    context its tokens see (positions max(0, start - W + 1) .. start - 1),
    the block's q, k, v and gate read and its output written (bf16)."""
    ctx = start if window == 0 else min(start, window - 1)
    io = batch * seq * d * 2 * (hq + hkv + hkv + hq + hq)
    return batch * ctx * kv_bytes_per_token(hkv, d, elem_bytes) + io


def decode_visible_history(kv_len: int, window: int) -> int:
    """Cached entries one decode query reads (the new token excluded)."""
    if window == 0:
        return kv_len - 1
    return min(kv_len, window) - 1


def decode_kv_bytes(hkv: int, d: int, lengths, window: int, elem_bytes: int = 2) -> int:
    """Bytes of cached K and V one decode step reads, summed over sequences."""
    per = kv_bytes_per_token(hkv, d, elem_bytes)
    return sum(decode_visible_history(int(n), window) * per for n in lengths)


def decode_scale_bytes(hkv: int, lengths, window: int, page_tokens: int) -> int:
    """Bytes of float32 K and V scales an FP8 decode step reads: one pair per
    (page, head) holding visible history (paged) or per (sequence, head)."""
    if page_tokens == 0:
        return len(lengths) * hkv * 8
    return sum(-(-decode_visible_history(int(n), window) // page_tokens) * hkv * 8 for n in lengths)


def decode_io_bytes(hq: int, hkv: int, d: int, batch: int, elem_bytes: int = 2) -> int:
    """Per-step bytes outside the cache: q, gate, new k and v read, output
    written (bf16), new k and v appended (cache element size)."""
    return batch * d * (2 * (hq + hq + hkv + hkv + hq) + 2 * hkv * elem_bytes)


def decode_flops(hq: int, d: int, lengths, window: int) -> int:
    return sum(flops_per_pair(hq, d) * min(int(n), window if window else int(n))
               for n in lengths)


def decode_attention_flops_per_token(hq: int, d: int, n_global: int, n_local: int,
                                     context: int, window: int = 2048) -> int:
    """A(c): attention FLOPs of one decoded token over a whole layer stack."""
    return flops_per_pair(hq, d) * (n_global * context + n_local * min(context, window))


def kv_cache_bytes(hkv: int, d: int, n_global: int, n_local: int, context: int,
                   window: int = 2048, elem_bytes: int = 2) -> int:
    """KV(c) = n_global * b * c + n_local * b * min(c, W)."""
    b = kv_bytes_per_token(hkv, d, elem_bytes)
    return n_global * b * context + n_local * b * min(context, window)


def block_flops(hq: int, hkv: int, d: int, hidden: int, batch: int, seq: int, window: int) -> int:
    """The attention half of a decoder block: the q/k/v/gate and o projections
    (2 flops per multiply-add) plus the layer's attention flops."""
    rows = batch * seq
    proj = 2 * rows * hidden * (2 * hq + 2 * hkv) * d + 2 * rows * hq * d * hidden
    return proj + prefill_flops(hq, d, batch, seq, window)

