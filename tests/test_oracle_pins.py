"""Pins for the CPU oracle: each oracle function checked against something other
than itself -- fold identities the pages state, brute force on tiny inputs,
closed forms, invariants, and torch CPU library routines.  CPU only.

RT = reading note on "Running VLAs at Real-time Speed" (Ma et al.,
arXiv:2510.26742v1); PS = AREX Feed article on PhysisServe.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from conftest import f32_tree, shape_kwargs

F64 = np.float64
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- P1: RMSNorm fold (RT §4.1)
def test_rmsnorm_gain_fold_identity():
    r = rng(1)
    x = r.standard_normal((7, 48))
    g = r.uniform(0.5, 1.5, 48)
    W = r.standard_normal((48, 20))
    xhat = oracle.rms_norm(x, np.ones(48), 1e-6, F64)
    lhs = oracle.rms_norm(x, g, 1e-6, F64) @ W          # (x_hat * g) W
    rhs = xhat @ (np.diag(g) @ W)                        # x_hat [diag(g) W]
    assert rel(lhs, rhs) < 1e-12


# ---------------------------------------------------------------- P2: fused QKV (RT §4.3)
def test_fused_qkv_concat_split_identity():
    r = rng(2)
    a = r.standard_normal((9, 32))
    Wq, Wk, Wv = (r.standard_normal((32, n)) for n in (64, 16, 16))
    fused = a @ np.concatenate([Wq, Wk, Wv], axis=1)
    assert rel(fused[:, :64], a @ Wq) < 1e-12
    assert rel(fused[:, 64:80], a @ Wk) < 1e-12
    assert rel(fused[:, 80:], a @ Wv) < 1e-12


# ---------------------------------------------------------------- P3: action/time fold (RT §4.2)
def test_action_time_fold_identity():
    r = rng(3)
    A, D, N = 8, 16, 5
    a = r.standard_normal((N, A))
    W1, b1 = r.standard_normal((A, D)), r.standard_normal(D)
    W2, b2 = r.standard_normal((2 * D, D)), r.standard_normal(D)
    for t in (1.0, 0.7, 0.1):
        tau = oracle.time_embedding(t, D)
        unfused = np.concatenate([a @ W1 + b1, np.broadcast_to(tau, (N, D))], 1) @ W2 + b2
        W2a, W2t = W2[:D], W2[D:]
        folded = a @ (W1 @ W2a) + (b1 @ W2a + tau @ W2t + b2)
        assert rel(unfused, folded) < 1e-12


# ---------------------------------------------------------------- P4: RMSNorm / SiLU vs torch
@pytest.mark.parametrize("scale", [1.0, 1e-3])
def test_rms_norm_matches_torch(scale):
    r = rng(4)
    x = r.standard_normal((5, 64)) * scale   # small scale makes eps visible
    g = r.uniform(0.5, 1.5, 64)
    ref = F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    assert rel(oracle.rms_norm(x, g, 1e-6, F64), ref) < 1e-13


def test_silu_matches_torch_and_zero():
    z = np.linspace(-20, 20, 401)
    assert rel(oracle.silu(z, F64), F.silu(torch.from_numpy(z)).numpy()) < 1e-14
    assert oracle.silu(np.zeros(3), F64).tolist() == [0.0, 0.0, 0.0]


# ---------------------------------------------------------------- P5: attention
def brute_attention(q, k, v):
    """Pure-Python loops: softmax over keys of q.k/sqrt(d), GQA map h -> h*Hkv//Hq."""
    T, Hq, d = q.shape
    L, Hkv, _ = k.shape
    out = np.zeros((T, Hq, d))
    for t in range(T):
        for h in range(Hq):
            g = h * Hkv // Hq
            logits = [sum(q[t, h, i] * k[j, g, i] for i in range(d)) / math.sqrt(d)
                      for j in range(L)]
            mx = max(logits)
            w = [math.exp(s - mx) for s in logits]
            z = sum(w)
            for i in range(d):
                out[t, h, i] = sum(w[j] * v[j, g, i] for j in range(L)) / z
    return out


@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (4, 2), (3, 3)])
def test_attention_brute_force(Hq, Hkv):
    r = rng(5)
    q = r.standard_normal((3, Hq, 4))
    k = r.standard_normal((8, Hkv, 4))
    v = r.standard_normal((8, Hkv, 4))
    assert rel(oracle.attention(q, k, v, F64), brute_attention(q, k, v)) < 1e-12


@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (4, 2), (6, 6)])
def test_attention_matches_torch_sdpa(Hq, Hkv):
    r = rng(6)
    T, L, d = 11, 29, 32
    q = r.standard_normal((T, Hq, d))
    k = r.standard_normal((L, Hkv, d))
    v = r.standard_normal((L, Hkv, d))
    rep = Hq // Hkv
    tq = torch.from_numpy(q).permute(1, 0, 2)                          # [Hq, T, d]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(rep, 0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(rep, 0)
    ref = F.scaled_dot_product_attention(tq, tk, tv).permute(1, 0, 2).numpy()
    assert rel(oracle.attention(q, k, v, F64), ref) < 1e-12


def test_attention_closed_forms():
    r = rng(7)
    d = 16
    q = r.standard_normal((4, 2, d))
    # a single key: the output is that key's value
    k1, v1 = r.standard_normal((1, 1, d)), r.standard_normal((1, 1, d))
    o = oracle.attention(q, k1, v1, F64)
    assert rel(o, np.broadcast_to(v1[0, 0], o.shape)) < 1e-14
    # identical keys: the output is the mean of the values
    kk = np.broadcast_to(r.standard_normal(d), (9, 1, d)).copy()
    vv = r.standard_normal((9, 1, d))
    o = oracle.attention(q, kk, vv, F64)
    assert rel(o, np.broadcast_to(vv[:, 0].mean(0), o.shape)) < 1e-12
    # one dominant logit picks its value
    kd = r.standard_normal((6, 1, d)) * 1e-3
    qd = np.zeros((1, 1, d)); qd[0, 0, 0] = 1.0
    kd[4, 0, 0] = 1e3
    o = oracle.attention(qd, kd, vv[:6], F64)
    assert rel(o[0, 0], vv[4, 0]) < 1e-12


def test_attention_key_permutation_invariance():
    """No mask: reordering the cached keys/values jointly changes nothing."""
    r = rng(8)
    q = r.standard_normal((5, 4, 8))
    k = r.standard_normal((13, 2, 8))
    v = r.standard_normal((13, 2, 8))
    perm = r.permutation(13)
    assert rel(oracle.attention(q, k[perm], v[perm], F64), oracle.attention(q, k, v, F64)) < 1e-12


# ---------------------------------------------------------------- P6: RoPE invariants
def test_rope_position_zero_is_identity():
    u = rng(9).standard_normal((1, 3, 64))
    c, s = oracle.rope_tables([0], 64, 10000.0, F64)
    assert np.array_equal(oracle.apply_rope(u, c, s, F64), u)


def test_rope_matches_complex_rotation():
    """Pair (u_j, u_{j+d/2}) as the complex number u_j + i u_{j+d/2}, multiplied
    by exp(i p theta_j) with theta_j = base^(-2j/d)."""
    r = rng(10)
    d, T = 32, 6
    pos = np.array([0, 1, 5, 100, 777, 6239])
    u = r.standard_normal((T, 2, d))
    c, s = oracle.rope_tables(pos, d, 10000.0, F64)
    got = oracle.apply_rope(u, c, s, F64)
    zc = u[..., : d // 2] + 1j * u[..., d // 2:]
    theta = 10000.0 ** (-np.arange(d // 2) * 2.0 / d)
    rot = zc * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    ref = np.concatenate([rot.real, rot.imag], -1)
    assert rel(got, ref) < 1e-12


def test_rope_preserves_pair_norms_and_relative_position():
    r = rng(11)
    d = 64
    qv, kv = r.standard_normal(d), r.standard_normal(d)

    def rot(vec, p):
        c, s = oracle.rope_tables([p], d, 10000.0, F64)
        return oracle.apply_rope(vec[None, None, :], c, s, F64)[0, 0]

    a = rot(qv, 37)
    half = d // 2
    assert rel(a[:half] ** 2 + a[half:] ** 2, qv[:half] ** 2 + qv[half:] ** 2) < 1e-12
    base = rot(qv, 50) @ rot(kv, 20)
    for shift in (1, 13, 500):
        assert abs(rot(qv, 50 + shift) @ rot(kv, 20 + shift) - base) < 1e-9 * max(1, abs(base))


# ---------------------------------------------------------------- P7: gated FFN brute force
def test_gated_ffn_brute_force():
    r = rng(12)
    b = r.standard_normal((2, 3))
    Wg, Wu, Wd = r.standard_normal((3, 4)), r.standard_normal((3, 4)), r.standard_normal((4, 3))
    ref = np.zeros((2, 3))
    for m, n in itertools.product(range(2), range(3)):
        acc = 0.0
        for j in range(4):
            gsum = sum(b[m, i] * Wg[i, j] for i in range(3))
            usum = sum(b[m, i] * Wu[i, j] for i in range(3))
            acc += gsum / (1 + math.exp(-gsum)) * usum * Wd[j, n]
        ref[m, n] = acc
    assert rel(oracle.gated_ffn(b, Wg, Wu, Wd, F64), ref) < 1e-13


# ---------------------------------------------------------------- P8: Euler closed forms
def test_euler_constant_velocity():
    a0 = rng(13).standard_normal((63, 32))
    c = rng(14).standard_normal((63, 32))
    sched = synth.flow_schedule(synth.FLOW)
    a, vs = oracle.euler_integrate(a0, sched, lambda a, s, t: c, F64)
    assert len(vs) == 10
    assert rel(a, a0 - c) < 1e-13


def test_euler_linear_velocity_closed_form():
    facts = json.load(open(GOLDEN))
    a0 = rng(15).standard_normal((63, 32))
    sched = synth.flow_schedule(synth.FLOW)
    a, _ = oracle.euler_integrate(a0, sched, lambda a, s, t: a, F64)
    assert rel(a, facts["euler_linear_factor_10"]["value"] * a0) < 1e-12


def test_euler_sees_the_schedule_times():
    seen = []
    sched = synth.flow_schedule(synth.FLOW)
    oracle.euler_integrate(np.zeros(2), sched, lambda a, s, t: (seen.append(t), a)[1], F64)
    assert seen == pytest.approx([1.0, 0.9, 0.8, 0.7, 0.6, 0.5, 0.4, 0.3, 0.2, 0.1], abs=1e-15)


# ---------------------------------------------------------------- time embedding
def test_time_embedding_properties():
    e0 = oracle.time_embedding(0.0, 1024)
    assert np.array_equal(e0, np.concatenate([np.zeros(512), np.ones(512)]))
    for t in (0.1, 0.5, 1.0):
        e = oracle.time_embedding(t, 1024)
        assert rel(e[:512] ** 2 + e[512:] ** 2, np.ones(512)) < 1e-15
        assert e[0] == pytest.approx(math.sin(t), abs=1e-16)          # omega_0 = 1
        assert e[511] == pytest.approx(math.sin(t * 10000.0 ** (-511 / 512)), abs=1e-16)


# ---------------------------------------------------------------- P9: shape reading vs the pages
def test_parameter_counts_match_pages():
    facts = json.load(open(GOLDEN))
    s = synth.AE_BLOCK
    D, F_, qd, kd = s.hidden, s.ffn, s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim
    per_layer = D * qd + 2 * D * kd + qd * D + 3 * D * F_
    assert per_layer == 17_301_504
    total = facts["ae_layers"]["value"] * per_layer
    p = facts["ae_params_approx"]
    assert abs(total - p["value"]) / p["value"] < p["rel_tol"]
    assert synth.FLOW.n_actions + 1 == facts["chunk_positions"]["value"]
    assert synth.FLOW.n_layers == facts["ae_layers"]["value"]
    assert synth.FLOW.n_steps == facts["denoise_steps"]["value"]
    assert synth.FLOW.action_dim == facts["action_dim"]["value"]
    b = synth.BATCHED
    qd = b.n_q_heads * b.head_dim
    bytes5 = 2 * (b.hidden * 3 * qd + qd * b.hidden + 3 * b.hidden * b.ffn)
    q = facts["batched_block_bytes_approx"]
    assert abs(bytes5 - q["value"]) / q["value"] < q["rel_tol"]


# ---------------------------------------------------------------- block-level pins
def torch_block(x, w, kp, vp, Hq, Hkv, d, base, eps):
    """The block re-composed from torch CPU library primitives (float64)."""
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    x = t(x)
    T, D = x.shape
    P = kp.shape[0]
    a = F.rms_norm(x, (D,), t(w["g_attn"]), eps)
    q = (a @ t(w["w_q"])).view(T, Hq, d)
    k = (a @ t(w["w_k"])).view(T, Hkv, d)
    v = (a @ t(w["w_v"])).view(T, Hkv, d)
    pos = torch.arange(P, P + T, dtype=torch.float64)
    inv = base ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    ang = pos[:, None] * inv[None, :]
    cos, sin = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]

    def rope(u):  # complex multiply on half-split pairs
        z = torch.complex(u[..., : d // 2], u[..., d // 2:]) * torch.complex(cos, sin)
        return torch.cat([z.real, z.imag], -1)

    q, k = rope(q), rope(k)
    K = torch.cat([t(kp), k], 0).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    V = torch.cat([t(vp), v], 0).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    o = F.scaled_dot_product_attention(q.permute(1, 0, 2), K, V).permute(1, 0, 2).reshape(T, Hq * d)
    h = x + o @ t(w["w_o"])
    b = F.rms_norm(h, (D,), t(w["g_ffn"]), eps)
    y = h + (F.silu(b @ t(w["w_gate"])) * (b @ t(w["w_up"]))) @ t(w["w_down"])
    return y.numpy(), k.numpy(), v.numpy()


@pytest.mark.parametrize("shape", [synth.TINY, synth.small_shape()], ids=lambda s: s.name)
def test_block_matches_torch_recomposition(shape):
    case = synth.block_case(shape)
    w = f32_tree(case["weights"])
    st = f32_tree(case["streams"][0])
    y, k, v = oracle.block_forward(st["x"], w, st["k_prefix"], st["v_prefix"], dtype=F64,
                                   **shape_kwargs(shape))
    ty, tk, tv = torch_block(st["x"], w, st["k_prefix"], st["v_prefix"], shape.n_q_heads,
                             shape.n_kv_heads, shape.head_dim, shape.rope_base, shape.rms_eps)
    assert rel(y, ty) < 1e-12 and rel(k, tk) < 1e-12 and rel(v, tv) < 1e-12


def test_block_fp32_agrees_with_fp64_twin():
    shape = synth.TINY
    case = synth.block_case(shape)
    w = f32_tree(case["weights"])
    st = f32_tree(case["streams"][0])
    out32 = oracle.block_forward(st["x"], w, st["k_prefix"], st["v_prefix"], **shape_kwargs(shape))
    out64 = oracle.block_forward(st["x"], w, st["k_prefix"], st["v_prefix"], dtype=F64,
                                 **shape_kwargs(shape))
    for a, b in zip(out32, out64):
        assert a.dtype == np.float32
        assert rel(a, b) < 1e-5


def test_block_rows_subset_matches_full():
    shape = synth.small_shape()
    case = synth.block_case(shape)
    w = f32_tree(case["weights"])
    st = f32_tree(case["streams"][1])
    kw = shape_kwargs(shape)
    y, k, v = oracle.block_forward(st["x"], w, st["k_prefix"], st["v_prefix"], dtype=F64, **kw)
    rows = [0, 5, 36]
    ys, ks, vs = oracle.block_forward(st["x"], w, st["k_prefix"], st["v_prefix"], rows=rows,
                                      dtype=F64, **kw)
    assert rel(ys, y[rows]) < 1e-13 and np.array_equal(ks, k) and np.array_equal(vs, v)


def test_block_residual_identity_when_projections_vanish():
    """W_o = 0 and W_down = 0 leave only the two residual paths: y = x."""
    shape = synth.TINY
    case = synth.block_case(shape)
    w = dict(f32_tree(case["weights"]))
    w["w_o"] = np.zeros_like(w["w_o"])
    w["w_down"] = np.zeros_like(w["w_down"])
    st = f32_tree(case["streams"][0])
    y, _, _ = oracle.block_forward(st["x"], w, st["k_prefix"], st["v_prefix"], dtype=F64,
                                   **shape_kwargs(shape))
    assert np.array_equal(y, st["x"].astype(F64))


# ---------------------------------------------------------------- flow head pins
def test_suffix_embed_matches_torch_recomposition():
    flow = synth.FLOW
    h = f32_tree(synth.flow_head_weights(flow))
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    for tt in (1.0, 0.3):
        X = oracle.suffix_embed(h["noise"], h["state"], tt, h, F64)
        u = F.linear(t(h["noise"]), t(h["w1"]).T, t(h["b1"]))
        tau = t(oracle.time_embedding(tt, 1024)).expand(63, 1024)
        z = F.silu(F.linear(torch.cat([u, tau], 1), t(h["w2"]).T, t(h["b2"])))
        e_act = F.linear(z, t(h["w3"]).T, t(h["b3"]))
        e_state = F.linear(t(h["state"])[None], t(h["ws"]).T, t(h["bs"]))
        assert rel(X, torch.cat([e_state, e_act]).numpy()) < 1e-12


def test_velocity_head_matches_torch():
    flow = synth.FLOW
    h = f32_tree(synth.flow_head_weights(flow))
    X = rng(16).standard_normal((64, 1024))
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    ref = F.linear(F.rms_norm(t(X[1:]), (1024,), t(h["g_f"]), 1e-6), t(h["w_out"]).T, t(h["b_out"]))
    assert rel(oracle.velocity_head(X, h, 1e-6, F64), ref.numpy()) < 1e-12


@pytest.mark.slow
def test_flow_fp32_agrees_with_fp64_twin_two_layers():
    flow = synth.FLOW
    case = synth.flow_case(flow, n_layers=2)
    head = f32_tree(case["head"])
    layers = [f32_tree(l) for l in case["layers"]]
    kw = shape_kwargs(flow.block)
    a32, _ = oracle.flow_denoise(head["noise"], head["state"], case["schedule"], layers, head,
                                 n_layers=2, **kw)
    a64, _ = oracle.flow_denoise(head["noise"], head["state"], case["schedule"], layers, head,
                                 n_layers=2, dtype=F64, **kw)
    assert rel(a32, a64) < 1e-4


# ---------------------------------------------------------------- loop composition (RT §2, §4.2)
# A small action-expert stack: distinct weights and cached prefixes per layer,
# a state token plus 7 action tokens of width 8, three Euler evaluations.
LOOP_SMALL = synth.FlowShape(
    "flow_small_pin",
    synth.BlockShape("flow_small_layer", 128, 256, 4, 1, 32, 1, 8, 20, 4242),
    n_layers=2, n_steps=3, n_actions=7, action_dim=8, seed=4242)


def torch_loop(case, flow):
    """The denoise loop re-composed in float64 from torch CPU primitives: the
    embedding with F.linear / F.silu and the state token in row 0, each layer
    through torch_block with its own weights and its own cached prefix, the
    velocity as F.rms_norm + F.linear on the action rows X[1:], and explicit
    Euler with dt = t_{s+1} - t_s (t_n = 0)."""
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    h = f32_tree(case["head"])
    layers = [f32_tree(l) for l in case["layers"]]
    b = flow.block
    D = b.hidden
    sched = [float(v) for v in case["schedule"]] + [0.0]
    a = t(h["noise"])
    for s in range(flow.n_steps):
        u = F.linear(a, t(h["w1"]).T, t(h["b1"]))
        tau = t(oracle.time_embedding(sched[s], D)).expand(flow.n_actions, D)
        z = F.silu(F.linear(torch.cat([u, tau], 1), t(h["w2"]).T, t(h["b2"])))
        e_act = F.linear(z, t(h["w3"]).T, t(h["b3"]))
        e_state = F.linear(t(h["state"])[None], t(h["ws"]).T, t(h["bs"]))
        X = torch.cat([e_state, e_act], 0).numpy()
        for lw in layers:
            X, _, _ = torch_block(X, lw, lw["k_prefix"], lw["v_prefix"], b.n_q_heads,
                                  b.n_kv_heads, b.head_dim, b.rope_base, b.rms_eps)
        v = F.linear(F.rms_norm(t(X[1:]), (D,), t(h["g_f"]), b.rms_eps), t(h["w_out"]).T,
                     t(h["b_out"]))
        a = a + (sched[s + 1] - sched[s]) * v
    return a.numpy()


def oracle_loop(case, flow, layers=None):
    h = f32_tree(case["head"])
    ls = [f32_tree(l) for l in case["layers"]] if layers is None else layers
    a, _ = oracle.flow_denoise(h["noise"], h["state"], case["schedule"], ls, h, dtype=F64,
                               **shape_kwargs(flow.block))
    return a


def test_flow_loop_matches_torch_recomposition():
    case = synth.flow_case(LOOP_SMALL)
    assert rel(oracle_loop(case, LOOP_SMALL), torch_loop(case, LOOP_SMALL)) < 1e-12


@pytest.mark.slow
def test_flow_loop_matches_torch_recomposition_action_expert_shape():
    """Two layers of the action-expert stack (hidden 1024, 768 cached keys per
    layer) over the first three times of the ten-step schedule."""
    flow = synth.FlowShape("flow_2x3", synth.FLOW.block, n_layers=2, n_steps=3,
                           n_actions=63, action_dim=32, seed=synth.FLOW.seed)
    case = dict(synth.flow_case(flow))
    assert rel(oracle_loop(case, flow), torch_loop(case, flow)) < 1e-12


def test_loop_pin_catches_planted_mistakes(monkeypatch):
    """Plausible composition mistakes, planted in the oracle's loop on the CPU,
    that the torch re-composition must reject."""
    flow = LOOP_SMALL
    case = synth.flow_case(flow)
    ref = torch_loop(case, flow)
    layers = [f32_tree(l) for l in case["layers"]]
    assert rel(oracle_loop(case, flow, layers), ref) < 1e-12

    # every layer reads layer 0's cached prefix
    shared = [dict(l, k_prefix=layers[0]["k_prefix"], v_prefix=layers[0]["v_prefix"])
              for l in layers]
    assert rel(oracle_loop(case, flow, shared), ref) > 1e-3
    # the layers run in the wrong order
    assert rel(oracle_loop(case, flow, layers[::-1]), ref) > 1e-3

    import oracle.flow as of

    # the velocity taken on X[:-1] (state row kept, last action row dropped)
    def vel_wrong_rows(X, head, eps, dtype=np.float32):
        Xa = np.asarray(X, dtype)[:-1]
        return of.rms_norm(Xa, head["g_f"], eps, dtype) @ np.asarray(head["w_out"], dtype) \
            + np.asarray(head["b_out"], dtype)

    with monkeypatch.context() as m:
        m.setattr(of, "velocity_head", vel_wrong_rows)
        assert rel(oracle_loop(case, flow, layers), ref) > 1e-3

    # Euler with the step's sign flipped (+|dt|)
    def euler_plus(a0, schedule, velocity, dtype=np.float32):
        a = np.asarray(a0, dtype)
        n = len(schedule)
        for s in range(n):
            t = float(schedule[s])
            t_next = float(schedule[s + 1]) if s + 1 < n else 0.0
            a = a + dtype(t - t_next) * np.asarray(velocity(a, s, t), dtype)
        return a, []

    with monkeypatch.context() as m:
        m.setattr(of, "euler_integrate", euler_plus)
        assert rel(oracle_loop(case, flow, layers), ref) > 1e-3

    # the state token appended last instead of first
    good_embed = of.suffix_embed

    def embed_state_last(actions, state, t, head, dtype=np.float32):
        X = good_embed(actions, state, t, head, dtype)
        return np.concatenate([X[1:], X[:1]], axis=0)

    with monkeypatch.context() as m:
        m.setattr(of, "suffix_embed", embed_state_last)
        assert rel(oracle_loop(case, flow, layers), ref) > 1e-3


# ---------------------------------------------------------------- planted mistakes are caught
def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in copies of oracle steps (on the CPU) and check
    that the library/brute-force pins above would reject each of them."""
    r = rng(17)
    q = r.standard_normal((3, 4, 8))
    k = r.standard_normal((10, 2, 8))
    v = r.standard_normal((10, 2, 8))
    good = brute_attention(q, k, v)

    def att_no_scale(q, k, v):
        return oracle.attention(q * math.sqrt(8), k, v, F64)

    def att_wrong_group(q, k, v):  # h % Hkv instead of h * Hkv // Hq
        return oracle.attention(q[:, [0, 2, 1, 3], :], k, v, F64)[:, [0, 2, 1, 3], :]

    assert rel(att_no_scale(q, k, v), good) > 1e-3
    assert rel(att_wrong_group(q, k, v), good) > 1e-3

    # RoPE with the rotation reversed passes relative-position invariance but
    # fails the complex-rotation pin.
    pos = np.array([3, 9])
    u = r.standard_normal((2, 1, 16))
    c, s = oracle.rope_tables(pos, 16, 10000.0, F64)
    wrong = oracle.apply_rope(u, c, -s, F64)
    zc = u[..., :8] + 1j * u[..., 8:]
    theta = 10000.0 ** (-np.arange(8) * 2.0 / 16)
    rot = zc * np.exp(1j * pos[:, None, None] * theta)
    assert rel(wrong, np.concatenate([rot.real, rot.imag], -1)) > 1e-3

    # RMSNorm without eps is caught at small input scale.
    x = r.standard_normal((2, 16)) * 1e-4
    ref = F.rms_norm(torch.from_numpy(x), (16,), None, eps=1e-6).numpy()
    no_eps = x / np.sqrt(np.mean(x * x, -1, keepdims=True))
    assert rel(no_eps, ref) > 1e-3
