"""fp64 oracle of the attention sub-block around the layer (test
infrastructure only; see the package doc).

One decoder block's attention half, in the order the deep dive gives it
(section 2.1 forward walk, section 5.1 for Glimmer, 5.2-5.3 for Spark):

    h = input_layernorm(x)                     centered RMSNorm, gain 1 + w, eps 1e-5
    q, k, v, g = h W_q^T, h W_k^T, h W_v^T, h W_g^T      no biases (section 3.2)
    o = the attention layer (oracle.prefill)   per-head QK-norm, RoPE, mask, o_norm, gate
    a = o W_o^T                                o_proj
    Glimmer: out = x + centered_rmsnorm(a, w_post, eps 1e-8)
    Spark:   out = alpha * x + beta * rmsnorm(a, eps 1e-8)   (norm-preserving residual gate)

with beta = sigmoid(g_res / T), alpha = sqrt(max(sigmoid(-g_res / T) (1 +
beta), 1e-3)), T = 0.3 (section 5.2).  Everything is float64 with no
intermediate rounding; the projections are single matmuls.  In decode the
layer is one decode step over the cache as stored (attention_block_decode).
"""
from __future__ import annotations

import numpy as np

from .attention import decode_one, prefill, rms_normalize, sigmoid


def centered_rmsnorm(x, w, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) times the gain (1 + w) (section 5.3)."""
    return rms_normalize(x, eps) * (1.0 + np.asarray(w, dtype=np.float64))


def residual_gate(x, f, g, temperature: float = 0.3, alpha_sq_floor: float = 1e-3) -> np.ndarray:
    """Spark's norm-preserving residual gate alpha * x + beta * f (section 5.2)."""
    w = np.asarray(g, dtype=np.float64) / temperature
    beta = sigmoid(w)
    alpha = np.sqrt(np.maximum(sigmoid(-w) * (1.0 + beta), alpha_sq_floor))
    return alpha * np.asarray(x, dtype=np.float64) + beta * np.asarray(f, dtype=np.float64)


def input_projections(x, weights: dict, layer):
    """h = input_layernorm(x) and its four projections for tokens x [T, hidden]:
    returns q, k, v, g as [T, Hq, D], [T, Hkv, D], [T, Hkv, D], [T, Hq, D]."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    hq, hkv, d = layer.hq, layer.hkv, layer.d
    h = centered_rmsnorm(x, weights["in_norm"], 1e-5)
    proj = h @ np.asarray(weights["w_qkvg"], dtype=np.float64).T
    q = proj[:, :hq * d].reshape(T, hq, d)
    k = proj[:, hq * d:(hq + hkv) * d].reshape(T, hkv, d)
    v = proj[:, (hq + hkv) * d:(hq + 2 * hkv) * d].reshape(T, hkv, d)
    g = proj[:, (hq + 2 * hkv) * d:].reshape(T, hq, d)
    return q, k, v, g


def block_output(x, o, weights: dict) -> np.ndarray:
    """o_proj of the layer's output o [n, Hq, D], then the post-attention norm
    and the residual with x [n, hidden]: Glimmer's sandwich norm and add, or
    Spark's weightless norm and residual gate."""
    x = np.asarray(x, dtype=np.float64)
    a = np.asarray(o, dtype=np.float64).reshape(x.shape[0], -1) @ np.asarray(weights["w_o"], dtype=np.float64).T
    if weights.get("residual_gate") is not None:
        f = rms_normalize(a, 1e-8)
        return residual_gate(x, f, weights["residual_gate"], weights.get("temperature", 0.3))
    return x + centered_rmsnorm(a, weights["post_norm"], 1e-8)


def attention_block(x, weights: dict, layer, positions=None, rows=None) -> np.ndarray:
    """The attention half of a decoder block on one sequence, x [T, hidden].

    weights: in_norm [hidden]; w_qkvg [(2 Hq + 2 Hkv) D, hidden] (rows: q,
    k, v, gate); w_o [hidden, Hq D]; post_norm [hidden] (Glimmer) or
    residual_gate [hidden] (Spark), temperature (default 0.3).  ``rows``
    selects output rows (every row's attention needs the keys of all rows up
    to it, so x holds rows 0 .. max(rows)).  Returns [n_rows, hidden]."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    q, k, v, g = input_projections(x, weights, layer)
    if rows is None:
        rows = np.arange(T)
    rows = np.asarray(rows, dtype=np.int64)
    o = prefill(q[rows], k, v, g[rows], layer, positions=positions, rows=rows)
    return block_output(x[rows], o, weights)


def attention_block_decode(x_new, weights: dict, layer, k_hist, v_hist, hist_start: int,
                           kv_len: int) -> np.ndarray:
    """One new token of one sequence through the block: x_new [hidden] at
    position kv_len - 1.  Its projections give q, k, v and the gate; the layer
    is one decode step (oracle.decode_one) over the cached history k_hist,
    v_hist [n, Hkv, D] of positions hist_start .. hist_start + n - 1, taken as
    stored, plus the token's own key and value.  Returns [hidden]."""
    x = np.asarray(x_new, dtype=np.float64)[None]
    q, k, v, g = input_projections(x, weights, layer)
    o = decode_one(q[0], k[0], v[0], g[0], k_hist, v_hist, hist_start, kv_len, layer)
    return block_output(x, o[None], weights)[0]
