"""Flow-matching action-expert loop: suffix embedding, block stack, velocity
head and Euler integration.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Unfused: the action
projection, the concatenation with the time embedding and the second linear
layer are computed as written, not pre-multiplied.

[RT] §2 / Fig. 4: an action expert denoises a 63-step action chunk (padded to
32 dims) over 10 flow-matching steps, reusing the prefix KV cache; 63 action
tokens plus one state token make 64 positions; the layer stack repeats 18x.
[RT] §4.2: the action linear projection is concatenated with the time encoding
and fed to another linear layer, followed by SiLU.
"""
from __future__ import annotations

import numpy as np

from .block import block_forward, rms_norm, silu


def _c(a, dtype):
    return np.asarray(a, dtype=dtype)


def time_embedding(t, dim):
    """Sinusoidal embedding of a scalar time t, float64.

    tau_j = sin(t w_j), tau_{dim/2 + j} = cos(t w_j), w_j = 10000^(-j/(dim/2)),
    j < dim/2, t unscaled.  Reading: the pages name a sinusoidal embedding of
    dim 1024 without its exact form; this is the plain transformer form.
    """
    half = dim // 2
    j = np.arange(half, dtype=np.float64)
    omega = np.power(10000.0, -j / half)
    ang = np.float64(t) * omega
    return np.concatenate([np.sin(ang), np.cos(ang)])


def suffix_embed(actions, state, t, head, dtype=np.float32):
    """Token embeddings of the action expert's chunk at time t.

    e_act = SiLU([a W1 + b1, tau(t)] W2 + b2) W3 + b3      (63 rows)
    e_state = state Ws + bs                               (1 row, index 0)
    Returns X = [e_state; e_act], [1 + N, D].
    W2 is [2D, D]: rows 0..D-1 act on the action branch, rows D..2D-1 on
    tau(t).  Reading: W3 (the linear after SiLU) completes the chain the note
    describes up to SiLU.
    """
    a = _c(actions, dtype)
    D = head["w1"].shape[1]
    u = a @ _c(head["w1"], dtype) + _c(head["b1"], dtype)
    tau = time_embedding(t, D).astype(dtype)
    cat = np.concatenate([u, np.broadcast_to(tau, u.shape)], axis=1)
    z = silu(cat @ _c(head["w2"], dtype) + _c(head["b2"], dtype), dtype)
    e_act = z @ _c(head["w3"], dtype) + _c(head["b3"], dtype)
    e_state = _c(state, dtype)[None, :] @ _c(head["ws"], dtype) + _c(head["bs"], dtype)
    return np.concatenate([e_state, e_act], axis=0)


def velocity_head(X, head, eps, dtype=np.float32):
    """v = RMSNorm(X[1:]) g_F W_out + b_out on the action rows (row 0 is the
    state token and produces no action)."""
    Xa = _c(X, dtype)[1:]
    return rms_norm(Xa, head["g_f"], eps, dtype) @ _c(head["w_out"], dtype) \
        + _c(head["b_out"], dtype)


def euler_integrate(a0, schedule, velocity, dtype=np.float32):
    """Explicit Euler over the evaluation times t_0 > t_1 > ... > t_{n-1}, ending
    at t_n = 0: a_{s+1} = a_s + (t_{s+1} - t_s) v(a_s, s, t_s).

    Reading of the schedule t = 1.0 -> 0.0 in uniform steps of 0.1: ten
    evaluations at t = 1.0, 0.9, ..., 0.1, step -0.1 each.  The step is formed
    in float64 from the schedule and then cast.
    Returns (a_n, [v_0 .. v_{n-1}]).
    """
    a = _c(a0, dtype)
    vs = []
    n = len(schedule)
    for s in range(n):
        t = float(schedule[s])
        t_next = float(schedule[s + 1]) if s + 1 < n else 0.0
        v = _c(velocity(a, s, t), dtype)
        vs.append(v)
        a = a + dtype(t_next - t) * v
    return a, vs


def flow_denoise(noise, state, schedule, layers, head, *, n_q_heads, n_kv_heads, head_dim,
                 rope_base, eps, dtype=np.float32, n_layers=None):
    """The action expert's denoise loop.

    For each evaluation time: X = suffix_embed(a, state, t); X = block_l(X)
    for every layer l with its own weights and its own cached prefix K/V (the
    same cache at every step, [RT] §2); v = velocity_head(X); Euler step.
    Returns (a_final, per-step velocities).
    """
    L = len(layers) if n_layers is None else n_layers

    def velocity(a, s, t):
        X = suffix_embed(a, state, t, head, dtype)
        for l in range(L):
            lw = layers[l]
            X, _, _ = block_forward(X, lw, lw["k_prefix"], lw["v_prefix"],
                                    n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                                    head_dim=head_dim, rope_base=rope_base, eps=eps,
                                    dtype=dtype)
        return velocity_head(X, head, eps, dtype)

    return euler_integrate(noise, schedule, velocity, dtype)
