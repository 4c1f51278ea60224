"""One transformer-block stage on a chunk of query tokens over cached K/V.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain NumPy, unfused:
separate gains, separate Q/K/V projections, explicit RoPE, per-head softmax.

Block topology (pre-norm, two residual adds, no biases inside the block) is
the standard Gemma-style layer the [RT] note decomposes in its Fig. 4
(normalisation, residual, activation) with the gated FFN of its §5.
"""
from __future__ import annotations

import numpy as np


def _c(a, dtype):
    return np.asarray(a, dtype=dtype)


def rms_norm(x, g, eps, dtype=np.float32):
    """RMSNorm with a multiplicative per-channel gain: x * (mean_j x_j^2 + eps)^-1/2 * g.

    [RT] §4.1: the normalisation depends on the input; the learnable gain g is
    a fixed per-channel scale (the part that may be folded into the next
    linear layer).  Reading: eps = 1e-6 and the gain form x_hat * g (not 1+g).
    """
    x = _c(x, dtype)
    g = _c(g, dtype)
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=dtype)
    r = dtype(1.0) / np.sqrt(ms + dtype(eps))
    return (x * r) * g


def rope_tables(positions, head_dim, base, dtype=np.float32):
    """cos/sin of p * theta_j, theta_j = base^(-2j/d), j < d/2; angles in float64.

    [RT] §4.3: the fixed position-encoding quantities are precomputed.
    Reading: half-split pairs (j, j + d/2), base 10000.
    """
    j = np.arange(head_dim // 2, dtype=np.float64)
    theta = np.power(np.float64(base), -2.0 * j / head_dim)
    ang = np.outer(np.asarray(positions, dtype=np.float64), theta)
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def apply_rope(u, cos, sin, dtype=np.float32):
    """Rotate pairs (u_j, u_{j+d/2}) by angle p*theta_j.

    u: [T, H, d]; cos, sin: [T, d/2].  (a, b) -> (a cos - b sin, a sin + b cos).
    """
    u = _c(u, dtype)
    half = u.shape[-1] // 2
    c = _c(cos, dtype)[:, None, :]
    s = _c(sin, dtype)[:, None, :]
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def attention(q, k, v, dtype=np.float32):
    """softmax(q_h K_g^T / sqrt(d)) V_g per query head h, g = floor(h * Hkv / Hq).

    q: [T, Hq, d]; k, v: [L, Hkv, d] (L = all keys: cached prefix then the
    chunk's own).  No mask: every query sees every key ([PS] a chunk reads the
    earlier chunks' KV; configs say the chunk attends causally-free over the
    prefix plus its own tokens).  The row maximum is subtracted before exp.
    """
    q = _c(q, dtype)
    k = _c(k, dtype)
    v = _c(v, dtype)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = dtype(1.0 / np.sqrt(np.float64(d)))
    out = np.empty((T, Hq, d), dtype=dtype)
    for h in range(Hq):
        g = (h * Hkv) // Hq
        s = (q[:, h, :] @ k[:, g, :].T) * scale
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True, dtype=dtype)
        out[:, h, :] = p @ v[:, g, :]
    return out


def silu(z, dtype=np.float32):
    """SiLU(z) = z / (1 + exp(-z))."""
    z = _c(z, dtype)
    return z / (dtype(1.0) + np.exp(-z))


def gated_ffn(b, w_gate, w_up, w_down, dtype=np.float32):
    """(SiLU(b W_g) * (b W_u)) W_d -- [RT] §5: two up-projections of the same
    input, SiLU activation, elementwise gate, down-projection."""
    b = _c(b, dtype)
    gate = b @ _c(w_gate, dtype)
    up = b @ _c(w_up, dtype)
    return (silu(gate, dtype) * up) @ _c(w_down, dtype)


def block_forward(x, w, k_prefix, v_prefix, *, n_q_heads, n_kv_heads, head_dim,
                  rope_base, eps, rows=None, dtype=np.float32):
    """One stage for one stream.

    x: [T, D] chunk; w: dict with g_attn [D], w_q [D, Hq d], w_k, w_v [D, Hkv d],
    w_o [Hq d, D], g_ffn [D], w_gate, w_up [D, F], w_down [F, D] ([in, out]
    layout); k_prefix, v_prefix: [P, Hkv, d] cached keys (already rotated) and
    values.  Chunk token t sits at position P + t.

    Steps: a = RMSNorm(x) g1; q, k, v = a W_q, a W_k, a W_v; RoPE on q and k;
    attention over [prefix ; own] keys; h = x + O W_o; b = RMSNorm(h) g2;
    y = h + FFN(b).

    ``rows`` (optional) restricts q and every per-row output to those chunk
    rows; k_new / v_new are always computed for all T tokens because every
    query attends to all of them.

    Returns (y [len(rows) or T, D], k_new [T, Hkv, d], v_new [T, Hkv, d]).
    """
    x = _c(x, dtype)
    T, D = x.shape
    P = k_prefix.shape[0]
    d = head_dim
    a = rms_norm(x, w["g_attn"], eps, dtype)                      # [T, D]
    k = (a @ _c(w["w_k"], dtype)).reshape(T, n_kv_heads, d)
    v = (a @ _c(w["w_v"], dtype)).reshape(T, n_kv_heads, d)
    sel = np.arange(T) if rows is None else np.asarray(rows)
    q = (a[sel] @ _c(w["w_q"], dtype)).reshape(len(sel), n_q_heads, d)
    cos_all, sin_all = rope_tables(P + np.arange(T), d, rope_base, dtype)
    k = apply_rope(k, cos_all, sin_all, dtype)
    q = apply_rope(q, cos_all[sel], sin_all[sel], dtype)
    K = np.concatenate([_c(k_prefix, dtype), k], axis=0)
    V = np.concatenate([_c(v_prefix, dtype), v], axis=0)
    o = attention(q, K, V, dtype).reshape(len(sel), n_q_heads * d)
    h = x[sel] + o @ _c(w["w_o"], dtype)
    b = rms_norm(h, w["g_ffn"], eps, dtype)
    y = h + gated_ffn(b, w["w_gate"], w["w_up"], w["w_down"], dtype)
    return y, k, v
