"""Seeded synthetic inputs for the block stage and the flow-matching loop.

This module is shared by the CPU oracle's tests, the GPU parity tests, the
bench and the smoke check.  It draws random numbers and rounds them to the
storage types; it holds none of the method's arithmetic (no normalisation,
projection, attention or embedding math).

Recipe (the same for every workload):
  * generator: numpy ``Generator(PCG64(seed))``;
  * float32 draws in the order the functions below list them, then
    round-to-nearest-even to bfloat16 for every matrix and activation;
  * weights ~ N(0, 0.02^2), RMSNorm gains ~ U(0.5, 1.5) kept in float32,
    activations and cached K/V ~ N(0, 1), flow-head biases ~ N(0, 0.02^2)
    kept in float32, noise and state ~ N(0, 1) in float32.

A bf16 tensor is returned as a pair: ``bits`` (uint16 storage, what the GPU
receives) and ``f32`` (the exact value of those bits widened to float32, what
the oracle receives).  Both describe identical numbers.
"""
from __future__ import annotations

import dataclasses
import functools

import numpy as np

WEIGHT_STD = 0.02
ROPE_BASE = 10000.0
RMS_EPS = 1e-6


# --------------------------------------------------------------------------
# storage-type helpers
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 storage bits to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Bf16:
    bits: np.ndarray  # uint16
    f32: np.ndarray   # float32, exactly the value of bits

    @property
    def shape(self):
        return self.bits.shape


def _bf16_normal(rng: np.random.Generator, shape, std: float) -> Bf16:
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    bits = f32_to_bf16_bits(v)
    del v
    return Bf16(bits, bf16_bits_to_f32(bits))


def _gain(rng: np.random.Generator, n: int) -> np.ndarray:
    return (np.float32(0.5) + rng.random(size=n, dtype=np.float32)).astype(np.float32)


def _f32_normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return v


# --------------------------------------------------------------------------
# workload shapes
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class BlockShape:
    name: str
    hidden: int        # D
    ffn: int           # F
    n_q_heads: int     # Hq
    n_kv_heads: int    # Hkv
    head_dim: int      # d
    batch: int         # B streams sharing one block's weights
    tokens: int        # T query tokens per stream (the chunk)
    prefix: int        # P cached prefix / history tokens per stream
    seed: int
    rope_base: float = ROPE_BASE
    rms_eps: float = RMS_EPS

    @property
    def rows(self) -> int:
        return self.batch * self.tokens


@dataclasses.dataclass(frozen=True)
class FlowShape:
    name: str
    block: BlockShape  # the layer shape (batch 1, tokens = n_actions + 1)
    n_layers: int
    n_steps: int
    n_actions: int
    action_dim: int
    seed: int


TINY = BlockShape("tiny_16tok", 256, 1024, 4, 1, 64, 1, 16, 64, 1001)
AE_BLOCK = BlockShape("ae_block_64tok", 1024, 4096, 8, 1, 256, 1, 64, 520, 1002)
FLOW = FlowShape(
    "flow_18x10",
    BlockShape("flow_layer", 1024, 4096, 8, 1, 256, 1, 64, 768, 1003),
    n_layers=18, n_steps=10, n_actions=63, action_dim=32, seed=1003)
VIDEO_DIT = BlockShape("video_dit_1560tok", 1536, 8960, 12, 12, 128, 1, 1560, 4680, 1004)
BATCHED = BlockShape("batched_8x880tok", 5120, 13824, 40, 40, 128, 8, 880, 2640, 1005)

BLOCK_SHAPES = {s.name: s for s in (TINY, AE_BLOCK, VIDEO_DIT, BATCHED)}


def small_shape(name="small_ragged", *, hidden=128, ffn=256, n_q_heads=4, n_kv_heads=2,
                head_dim=64, batch=2, tokens=37, prefix=45, seed=7) -> BlockShape:
    """A free-form shape for tests (ragged token counts, GQA, several streams)."""
    return BlockShape(name, hidden, ffn, n_q_heads, n_kv_heads, head_dim, batch,
                      tokens, prefix, seed)


# --------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------
LAYER_KEYS = ("g_attn", "w_q", "w_k", "w_v", "w_o", "g_ffn", "w_gate", "w_up", "w_down")


def layer_weights(shape: BlockShape, seed: int, qk_std: float | None = None) -> dict:
    """One block's raw (unfolded) weights in [in, out] layout.

    Draw order: g_attn, w_q, w_k, w_v, w_o, g_ffn, w_gate, w_up, w_down.
    ``qk_std`` overrides the std of w_q and w_k (the peaked-softmax variant).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    D, F = shape.hidden, shape.ffn
    qd = shape.n_q_heads * shape.head_dim
    kd = shape.n_kv_heads * shape.head_dim
    s_qk = WEIGHT_STD if qk_std is None else qk_std
    w = {}
    w["g_attn"] = _gain(rng, D)
    w["w_q"] = _bf16_normal(rng, (D, qd), s_qk)
    w["w_k"] = _bf16_normal(rng, (D, kd), s_qk)
    w["w_v"] = _bf16_normal(rng, (D, kd), WEIGHT_STD)
    w["w_o"] = _bf16_normal(rng, (qd, D), WEIGHT_STD)
    w["g_ffn"] = _gain(rng, D)
    w["w_gate"] = _bf16_normal(rng, (D, F), WEIGHT_STD)
    w["w_up"] = _bf16_normal(rng, (D, F), WEIGHT_STD)
    w["w_down"] = _bf16_normal(rng, (F, D), WEIGHT_STD)
    return w


def stream_activations(shape: BlockShape, seed: int, tokens: int | None = None,
                       prefix: int | None = None) -> dict:
    """One stream's chunk activations and cached K/V.

    Draw order: x [T, D], k_prefix [P, Hkv, d], v_prefix [P, Hkv, d].
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    T = shape.tokens if tokens is None else tokens
    P = shape.prefix if prefix is None else prefix
    kv = (P, shape.n_kv_heads, shape.head_dim)
    return {
        "x": _bf16_normal(rng, (T, shape.hidden), 1.0),
        "k_prefix": _bf16_normal(rng, kv, 1.0),
        "v_prefix": _bf16_normal(rng, kv, 1.0),
    }


@functools.lru_cache(maxsize=4)
def block_case(shape: BlockShape, qk_std: float | None = None) -> dict:
    """Weights (seed) and per-stream activations (seed*100 + b) for a block."""
    w = layer_weights(shape, shape.seed, qk_std)
    streams = [stream_activations(shape, shape.seed * 100 + b) for b in range(shape.batch)]
    return {"shape": shape, "weights": w, "streams": streams}


def flow_head_weights(flow: FlowShape) -> dict:
    """Flow head + noise + state, from Generator(PCG64(flow.seed)).

    Draw order: w1 [A, D], b1 [D], w2 [2D, D] (rows 0..D-1 multiply the action
    branch, rows D..2D-1 the time embedding), b2 [D], w3 [D, D], b3 [D],
    ws [A, D], bs [D], g_f [D], w_out [D, A], b_out [A], noise [N, A], state [A].
    """
    rng = np.random.Generator(np.random.PCG64(flow.seed))
    D, A, N = flow.block.hidden, flow.action_dim, flow.n_actions
    h = {}
    h["w1"] = _bf16_normal(rng, (A, D), WEIGHT_STD)
    h["b1"] = _f32_normal(rng, D, WEIGHT_STD)
    h["w2"] = _bf16_normal(rng, (2 * D, D), WEIGHT_STD)
    h["b2"] = _f32_normal(rng, D, WEIGHT_STD)
    h["w3"] = _bf16_normal(rng, (D, D), WEIGHT_STD)
    h["b3"] = _f32_normal(rng, D, WEIGHT_STD)
    h["ws"] = _bf16_normal(rng, (A, D), WEIGHT_STD)
    h["bs"] = _f32_normal(rng, D, WEIGHT_STD)
    h["g_f"] = _gain(rng, D)
    h["w_out"] = _bf16_normal(rng, (D, A), WEIGHT_STD)
    h["b_out"] = _f32_normal(rng, A, WEIGHT_STD)
    h["noise"] = _f32_normal(rng, (N, A), 1.0)
    h["state"] = _f32_normal(rng, A, 1.0)
    return h


def flow_layer(flow: FlowShape, layer: int) -> dict:
    """Layer ``layer`` of the stack: weights from seed*100+layer, its own
    cached prefix K/V from seed*10000+layer."""
    w = layer_weights(flow.block, flow.seed * 100 + layer)
    rng = np.random.Generator(np.random.PCG64(flow.seed * 10000 + layer))
    kv = (flow.block.prefix, flow.block.n_kv_heads, flow.block.head_dim)
    w["k_prefix"] = _bf16_normal(rng, kv, 1.0)
    w["v_prefix"] = _bf16_normal(rng, kv, 1.0)
    return w


def flow_schedule(flow: FlowShape) -> np.ndarray:
    """Evaluation times t_s = (n - s) / n, s = 0..n-1, in float64."""
    n = flow.n_steps
    return np.array([(n - s) / n for s in range(n)], dtype=np.float64)


@functools.lru_cache(maxsize=2)
def flow_case(flow: FlowShape, n_layers: int | None = None) -> dict:
    L = flow.n_layers if n_layers is None else n_layers
    return {
        "flow": flow,
        "head": flow_head_weights(flow),
        "layers": [flow_layer(flow, l) for l in range(L)],
        "schedule": flow_schedule(flow),
    }


# --------------------------------------------------------------------------
# device copies (torch is imported lazily; used by GPU tests, bench and smoke)
# --------------------------------------------------------------------------
def to_device(value, device="cuda"):
    """Bf16 -> torch.bfloat16 tensor with the same bits; float arrays -> float32."""
    import torch
    if isinstance(value, Bf16):
        t = torch.from_numpy(np.ascontiguousarray(value.bits).view(np.int16)).view(torch.bfloat16)
        return t.to(device)
    if isinstance(value, np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(value, dtype=np.float32)).to(device)
    return value


def tree_to_device(d: dict, device="cuda") -> dict:
    return {k: to_device(v, device) for k, v in d.items()}


def bf16_tensor_to_f32(t) -> np.ndarray:
    """Exact float32 values of a torch.bfloat16 tensor (any device)."""
    import torch
    return t.detach().float().cpu().numpy()
