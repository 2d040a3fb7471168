"""fp64 oracle of the attention layer (test infrastructure only; see package doc).

Arrays use the layout [T, H, D] per sequence (a leading batch axis where
noted). Inputs may be any float array; they are widened to float64 first.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# Index logic
# ---------------------------------------------------------------------------

def layer_is_global(i: int, n_layers: int) -> bool:
    """Layer i of n_layers is a global (full-attention, NoPE) layer iff
    (L - 1 - i) mod 4 == 0.  Muse Spark Open deep dive, section 2.2, the
    layer-type equation."""
    return (n_layers - 1 - i) % 4 == 0


def global_layers(n_layers: int) -> list[int]:
    return [i for i in range(n_layers) if layer_is_global(i, n_layers)]


def visible_range(i: int, window: int) -> tuple[int, int]:
    """Inclusive range [lo, hi] of keys visible to query i.

    Local layer (window W > 0): i - W < j <= i, the query itself included
    (deep dive, section 3.4: the window of 2048 includes the query).  Global
    layer (W == 0): 0 <= j <= i."""
    if window < 0:
        raise ValueError("window must be >= 0")
    lo = 0 if window == 0 else max(0, i - window + 1)
    return lo, i


def bidirectional_range(p: int, window: int, last: int) -> tuple[int, int]:
    """Inclusive range [lo, hi] of key positions a block-diffusion drafter's
    query at position p sees (deep dive, section 8.2, step 4: the block
    attends without a causal mask): |p - j| < W in both directions on a
    layer with window W > 0, every key on a window-0 layer, and keys exist
    only up to the block's last position `last`."""
    if window < 0:
        raise ValueError("window must be >= 0")
    if window == 0:
        return 0, last
    return max(0, p - window + 1), min(last, p + window - 1)


def visible_mask(n: int, window: int) -> np.ndarray:
    """Boolean [n, n] mask, entry (i, j) true iff key j is visible to query i."""
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        lo, hi = visible_range(i, window)
        m[i, lo:hi + 1] = True
    return m


# ---------------------------------------------------------------------------
# Prologue: weightless QK-norm, query multiplier, RoPE
# ---------------------------------------------------------------------------

def rms_normalize(x, eps: float) -> np.ndarray:
    """Weightless RMSNorm over the last axis: x / sqrt(mean(x^2) + eps).
    Deep dive, section 3.2, step 2 (eps inside the square root)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps)


def rope_inv_freq(d: int, theta: float) -> np.ndarray:
    """Inverse frequencies theta**(-2j/d), j = 0 .. d/2 - 1 (the 'default'
    RoPE type, no scaling; deep dive, section 3.4)."""
    j = np.arange(d // 2, dtype=np.float64)
    return np.float64(theta) ** (-2.0 * j / d)


def rope_rotate(x, positions, theta: float) -> np.ndarray:
    """Rotate every head of x [T, H, D] by its token's position.

    Dimension j is paired with j + D/2 (rotate_half pairing) and turned by
    angle a = p * theta**(-2j/D):
        x_j       <- x_j cos a - x_{j+D/2} sin a
        x_{j+D/2} <- x_{j+D/2} cos a + x_j sin a
    Deep dive, section 3.4 (whole head rotated; pairing note)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    pos = np.asarray(positions, dtype=np.float64)
    if pos.ndim != 1 or pos.shape[0] != x.shape[0]:
        raise ValueError("positions must hold one entry per token (leading axis of x)")
    ang = pos[:, None] * rope_inv_freq(d, theta)[None, :]      # [T, D/2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def to_bf16(x) -> np.ndarray:
    """The bf16 value nearest to each entry (round to nearest, ties to even),
    reached through float32 as a float32 tensor cast to bfloat16 is: the
    float32 bits are rounded at bit 16."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (r.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def query_prologue(q, positions, layer, reference_rounding: bool = False):
    """q_hat = s * norm(q), then RoPE at the query's position if theta != 0.
    q [T, Hq, D], positions [T].  Deep dive, section 3.2 steps 2-4: normalize
    each head (fp32 in the reference, fp64 here), multiply only the query by
    qk_scale_factor, rotate (local layers only).

    reference_rounding (a flagged second mode, never the parity reference):
    round where the pages' reference implementation does (section 3.2
    implementation notes): the normalized query is cast back to bf16, and the
    product with qk_scale_factor (a float32 scalar) is bf16 again.  RoPE and
    everything after stay fp64."""
    qh = rms_normalize(q, layer.qk_eps)
    if reference_rounding:
        qh = to_bf16(to_bf16(qh) * np.float64(np.float32(layer.scale)))
    else:
        qh = qh * np.float64(layer.scale)
    if layer.theta != 0:
        qh = rope_rotate(qh, positions, layer.theta)
    return qh


def key_prologue(k, positions, layer, reference_rounding: bool = False):
    """k_hat = norm(k), then RoPE if theta != 0 (no multiplier on keys).
    k [T, Hkv, D], positions [T].  V is not touched.  reference_rounding:
    the normalized key is cast back to bf16 (see query_prologue)."""
    kh = rms_normalize(k, layer.qk_eps)
    if reference_rounding:
        kh = to_bf16(kh)
    if layer.theta != 0:
        kh = rope_rotate(kh, positions, layer.theta)
    return kh


def qk_prologue(q, k, positions, layer):
    """Both prologues with the same positions (q and k of the same tokens)."""
    return query_prologue(q, positions, layer), key_prologue(k, positions, layer)


# ---------------------------------------------------------------------------
# Attention core and epilogue
# ---------------------------------------------------------------------------

def logits_for_row(qh_row, kh_vis, group: int) -> np.ndarray:
    """Logits l[h, j] = q_hat[h] . k_hat[j, floor(h/G)] / sqrt(D).

    qh_row [Hq, D]; kh_vis [n, Hkv, D].  Returns [Hq, n]."""
    hq, d = qh_row.shape
    out = np.empty((hq, kh_vis.shape[0]), dtype=np.float64)
    for h in range(hq):
        out[h] = kh_vis[:, h // group, :] @ qh_row[h]
    return out / np.sqrt(np.float64(d))


def softmax(x, axis=-1) -> np.ndarray:
    """fp64 softmax with the maximum subtracted."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - np.max(x, axis=axis, keepdims=True))
    return e / np.sum(e, axis=axis, keepdims=True)


def attend_rows(qh_rows, row_index, kh, v, layer) -> np.ndarray:
    """Attention output o (before the epilogue) for selected query rows.

    qh_rows [n, Hq, D] are the prologue outputs of query rows row_index[n]
    (token indices within the sequence); kh, v [T', Hkv, D] hold keys and
    values of tokens 0 .. T'-1 with T' > max(row_index).  For each row i the
    visible keys are visible_range(i, W); the softmax of the logits weights
    the visible values (deep dive, section 3.2 step 5)."""
    kh = np.asarray(kh, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = layer.group
    out = np.empty(np.shape(qh_rows), dtype=np.float64)
    for r, i in enumerate(row_index):
        lo, hi = visible_range(int(i), layer.window)
        kv = kh[lo:hi + 1]
        vv = v[lo:hi + 1]
        w = softmax(logits_for_row(qh_rows[r], kv, g), axis=-1)   # [Hq, n]
        for h in range(layer.hq):
            out[r, h] = w[h] @ vv[:, h // g, :]
    return out


def sigmoid(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def output_epilogue(o, gate, layer) -> np.ndarray:
    """Spark: weightless RMSNorm of each head's D outputs (before the gate);
    both models: y = o * sigmoid(g), elementwise over the Hq*D channels.
    Deep dive, section 3.3 (order attention -> per-head o_norm -> gate)."""
    o = np.asarray(o, dtype=np.float64)
    if layer.out_norm:
        o = rms_normalize(o, layer.out_eps)
    return o * sigmoid(gate)


# ---------------------------------------------------------------------------
# Whole-layer entry points
# ---------------------------------------------------------------------------

def prefill(q, k, v, gate, layer, positions=None, rows=None, reference_rounding: bool = False) -> np.ndarray:
    """The layer on one sequence: q, gate [T, Hq, D]; k, v [T', Hkv, D].

    ``rows`` (token indices) selects the output rows; q and gate then hold
    only those rows, while k and v hold tokens 0 .. max(rows).  Positions
    default to the token index.  reference_rounding selects the flagged
    second mode of the prologues.  Returns y [n_rows, Hq, D] in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if rows is None:
        rows = np.arange(q.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    if positions is None:
        positions = np.arange(k.shape[0], dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    qh = query_prologue(q, positions[rows], layer, reference_rounding)
    kh = key_prologue(k, positions[:k.shape[0]], layer, reference_rounding)
    o = attend_rows(qh, rows, kh, v, layer)
    return output_epilogue(o, gate, layer)


def decode_one(q_new, k_new, v_new, gate, k_hist, v_hist, hist_start: int,
               kv_len: int, layer) -> np.ndarray:
    """One decode step of one sequence.

    q_new, gate [Hq, D]; k_new, v_new [Hkv, D] are the new token's raw
    projections, at position p = kv_len - 1 (kv_len counts the new token).
    k_hist, v_hist [n, Hkv, D] are cached entries for positions
    hist_start .. hist_start + n - 1, taken exactly as stored (keys already
    normalized and rotated, as the cache is written after norm and RoPE:
    deep dive, section 3.2 notes).  The query sees the cached positions in
    visible_range(p, W) minus p itself, plus its own freshly computed key.
    Returns y [Hq, D]."""
    p = kv_len - 1
    lo, _ = visible_range(p, layer.window)
    if hist_start > lo:
        raise ValueError("history does not cover the visible range")
    if hist_start + np.shape(k_hist)[0] < p:
        raise ValueError("history does not reach position p - 1")
    qh = query_prologue(np.asarray(q_new)[None], [p], layer)
    kh_new = key_prologue(np.asarray(k_new)[None], [p], layer)
    a = lo - hist_start
    b = p - hist_start
    keys = np.concatenate([np.asarray(k_hist, dtype=np.float64)[a:b], kh_new], axis=0)
    vals = np.concatenate([np.asarray(v_hist, dtype=np.float64)[a:b],
                           np.asarray(v_new, dtype=np.float64)[None]], axis=0)
    g = layer.group
    w = softmax(logits_for_row(qh[0], keys, g), axis=-1)
    o = np.empty((layer.hq, np.shape(q_new)[-1]), dtype=np.float64)
    for h in range(layer.hq):
        o[h] = w[h] @ vals[:, h // g, :]
    return output_epilogue(o, gate, layer)


def prefill_chunk(q, k, v, gate, k_hist, v_hist, hist_start: int, start: int,
                  layer, rows=None) -> np.ndarray:
    """A chunk of T new tokens of one sequence whose first ``start``
    positions are already cached (chunked prefill).

    q, gate [T, Hq, D] and k, v [T, Hkv, D] are the chunk's raw projections
    at positions start .. start + T - 1.  k_hist, v_hist [n, Hkv, D] are the
    cached entries of positions hist_start .. hist_start + n - 1, taken
    exactly as stored (keys already normalized and rotated, as decode reads
    them).  Chunk token t at position P = start + t sees the positions in
    visible_range(P, W): cached ones below ``start`` and the chunk's own from
    ``start`` to P, whose keys get the prologue at their positions.  ``rows``
    (chunk token indices) selects the output rows; q and gate then hold only
    those rows.  Returns y [n_rows, Hq, D] in float64."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T = k.shape[0]
    if rows is None:
        rows = np.arange(T)
    rows = np.asarray(rows, dtype=np.int64)
    positions = start + np.arange(T, dtype=np.int64)
    qh = query_prologue(q, positions[rows], layer)
    kh_new = key_prologue(k, positions, layer)
    k_hist = np.asarray(k_hist, dtype=np.float64)
    v_hist = np.asarray(v_hist, dtype=np.float64)
    g = layer.group
    o = np.empty(np.shape(qh), dtype=np.float64)
    for r, t in enumerate(rows):
        lo, hi = visible_range(int(start + t), layer.window)
        if lo < start and (lo < hist_start or hist_start + k_hist.shape[0] < start):
            raise ValueError("history does not cover the visible range")
        # keys and values of positions lo .. hi, cached ones first
        a = lo - hist_start
        c = start - hist_start
        keys = np.concatenate([k_hist[a:c] if lo < start else k_hist[:0], kh_new[max(lo - start, 0):t + 1]])
        vals = np.concatenate([v_hist[a:c] if lo < start else v_hist[:0], v[max(lo - start, 0):t + 1]])
        w = softmax(logits_for_row(qh[r], keys, g), axis=-1)
        for h in range(layer.hq):
            o[r, h] = w[h] @ vals[:, h // g, :]
    return output_epilogue(o, gate, layer)


def block_bidirectional(q, k, v, gate, k_hist, v_hist, hist_start: int, start: int,
                        layer, rows=None) -> np.ndarray:
    """Non-causal block attention of a block-diffusion drafter (deep dive,
    section 8.2, step 4): the T block tokens at positions start .. start +
    T - 1 are the queries; keys and values are the cached context entries
    below ``start`` (taken as stored) followed by the block's own keys and
    values (prologue at their positions).  No causal mask: key position j is
    visible to query position P iff |P - j| < W on a layer with window W
    (both directions), and always on a layer with W = 0; keys exist only up
    to the block's last position.

    Arguments as for prefill_chunk; the history must reach back to
    start + t - W + 1 for every row t.  Returns y [n_rows, Hq, D]."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T = k.shape[0]
    if rows is None:
        rows = np.arange(T)
    rows = np.asarray(rows, dtype=np.int64)
    positions = start + np.arange(T, dtype=np.int64)
    qh = query_prologue(q, positions[rows], layer)
    kh_new = key_prologue(k, positions, layer)
    k_hist = np.asarray(k_hist, dtype=np.float64)
    v_hist = np.asarray(v_hist, dtype=np.float64)
    last = start + T - 1
    g = layer.group
    o = np.empty(np.shape(qh), dtype=np.float64)
    for r, t in enumerate(rows):
        lo, hi = bidirectional_range(int(start + t), layer.window, last)
        if lo < start and (lo < hist_start or hist_start + k_hist.shape[0] < start):
            raise ValueError("history does not cover the visible range")
        a = lo - hist_start
        c = start - hist_start
        keys = np.concatenate([k_hist[a:c] if lo < start else k_hist[:0], kh_new[max(lo - start, 0):hi - start + 1]])
        vals = np.concatenate([v_hist[a:c] if lo < start else v_hist[:0], v[max(lo - start, 0):hi - start + 1]])
        w = softmax(logits_for_row(qh[r], keys, g), axis=-1)
        for h in range(layer.hq):
            o[r, h] = w[h] @ vals[:, h // g, :]
    return output_epilogue(o, gate, layer)

