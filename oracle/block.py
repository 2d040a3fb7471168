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
intermediate rounding; the projections are single matmuls.
"""
from __future__ import annotations

import numpy as np

from .attention import prefill, rms_normalize, sigmoid


def centered_rmsnorm(x, w, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) times the gain (1 + w) (section 5.3)."""
    return rms_normalize(x, eps) * (1.0 + np.asarray(w, dtype=np.float64))


def residual_gate(x, f, g, temperature: float = 0.3, alpha_sq_floor: float = 1e-3) -> np.ndarray:
    """Spark's norm-preserving residual gate alpha * x + beta * f (section 5.2)."""
    w = np.asarray(g, dtype=np.float64) / temperature
    beta = sigmoid(w)
    alpha = np.sqrt(np.maximum(sigmoid(-w) * (1.0 + beta), alpha_sq_floor))
    return alpha * np.asarray(x, dtype=np.float64) + beta * np.asarray(f, dtype=np.float64)


def attention_block(x, weights: dict, layer, positions=None, rows=None) -> np.ndarray:
    """The attention half of a decoder block on one sequence, x [T, hidden].

    weights: in_norm [hidden]; w_qkvg [(2 Hq + 2 Hkv) D, hidden] (rows: q,
    k, v, gate); w_o [hidden, Hq D]; post_norm [hidden] (Glimmer) or
    residual_gate [hidden] (Spark), temperature (default 0.3).  ``rows``
    selects output rows (every row's attention needs the keys of all rows up
    to it, so x holds rows 0 .. max(rows)).  Returns [n_rows, hidden]."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    hq, hkv, d = layer.hq, layer.hkv, layer.d
    h = centered_rmsnorm(x, weights["in_norm"], 1e-5)
    proj = h @ np.asarray(weights["w_qkvg"], dtype=np.float64).T
    q = proj[:, :hq * d].reshape(T, hq, d)
    k = proj[:, hq * d:(hq + hkv) * d].reshape(T, hkv, d)
    v = proj[:, (hq + hkv) * d:(hq + 2 * hkv) * d].reshape(T, hkv, d)
    g = proj[:, (hq + 2 * hkv) * d:].reshape(T, hq, d)
    if rows is None:
        rows = np.arange(T)
    rows = np.asarray(rows, dtype=np.int64)
    o = prefill(q[rows], k, v, g[rows], layer, positions=positions, rows=rows)
    a = o.reshape(len(rows), hq * d) @ np.asarray(weights["w_o"], dtype=np.float64).T
    if weights.get("residual_gate") is not None:
        f = rms_normalize(a, 1e-8)
        return residual_gate(x[rows], f, weights["residual_gate"], weights.get("temperature", 0.3))
    return x[rows] + centered_rmsnorm(a, weights["post_norm"], 1e-8)
