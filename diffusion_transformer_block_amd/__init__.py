"""Python binding of libblk.so: the block stage over cached K/V and the
flow-matching denoise loop on MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/blk.h).  torch supplies device memory and
the current stream; there is no CPU fallback -- if libblk.so is not built or
no GPU is present, these functions raise.

Tensors:
  * bf16 tensors are torch.bfloat16 (passed by data pointer);
  * gains, biases, noise, state and actions are torch.float32;
  * weights are row-major [in, out].
"""
from __future__ import annotations

import ctypes
from ctypes import byref, c_double, c_int32, c_size_t, c_void_p

from ._lib import (BLK_EABORTED, BLK_EHIP, BLK_EINVAL, BLK_ESIZE, BLK_ESTATE, BLK_EUNSUPPORTED,
                   BLK_OK, EXPORTS, HEAD_FIELDS, LAYER_FIELDS, OPERATORS, WS_ABORT_OFFSET,
                   BlkConfig, BlkError, FlowHeadSrc, LayerSrc, check, load)

__all__ = ["BlkConfig", "BlkError", "make_config", "blk_prepare_weights", "blk_forward",
           "blk_forward_chunks",
           "blk_forward_noalloc", "NOALLOC_SCRATCH_BYTES", "prefix_prefill",
           "prefill_workspace_bytes",
           "flow_denoise", "blk_last_error", "blk_release", "blk_version", "EXPORTS",
           "blk_set_execution_mode", "EXEC_AUTO", "EXEC_PER_OPERATOR", "EXEC_PERSISTENT",
           "forward_workspace_bytes", "flow_workspace_bytes", "packed_bytes",
           "blk_set_operator_timing", "blk_operator_times", "OPERATORS", "probe_hbm_read",
           "blk_workspace_status", "WS_ABORT_OFFSET",
           "probe_mfma_bf16"]


def _torch():
    import torch
    return torch


def make_config(hidden, ffn, n_q_heads, n_kv_heads, head_dim, max_pos, rope_base=10000.0,
                rms_eps=1e-6) -> BlkConfig:
    return BlkConfig(hidden, ffn, n_q_heads, n_kv_heads, head_dim, max_pos, rope_base, rms_eps)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _layer_src(layer: dict) -> LayerSrc:
    return LayerSrc(*[_ptr(layer[n]) for n in LAYER_FIELDS])


def _head_src(head: dict) -> FlowHeadSrc:
    """head: dict with int ``n_actions`` and the blk_flow_head_src tensors;
    action_dim is w_out's column count."""
    return FlowHeadSrc(int(head["n_actions"]), int(head["w_out"].shape[1]),
                       *[_ptr(head[k]) for k in HEAD_FIELDS])


def packed_bytes(cfg: BlkConfig, n_layers: int, head: dict | None = None,
                 t_schedule=None) -> int:
    lib = load()
    nbytes = c_size_t(0)
    arr = (LayerSrc * max(n_layers, 1))()
    hs = _head_src(head) if head is not None else None
    ts = (c_double * len(t_schedule))(*t_schedule) if t_schedule is not None else None
    n_steps = len(t_schedule) if t_schedule is not None else 0
    check("blk_prepare_weights", lib.blk_prepare_weights(
        byref(cfg), arr, n_layers, byref(hs) if hs is not None else None, ts, n_steps, None,
        byref(nbytes), None))
    return nbytes.value


def blk_prepare_weights(cfg: BlkConfig, layers: list, head: dict | None = None,
                        t_schedule=None, stream=None, out=None):
    """Pack ``layers`` (dicts of device tensors named as in blk_layer_src) and an
    optional flow head (dict with ``n_actions`` and the blk_flow_head_src
    tensors) into one uint8 device tensor.  Keep the returned tensor alive while
    it is used; it is registered by address."""
    torch = _torch()
    lib = load()
    n_layers = len(layers)
    arr = (LayerSrc * max(n_layers, 1))(*[_layer_src(l) for l in layers])
    hs = _head_src(head) if head is not None else None
    ts = (c_double * len(t_schedule))(*[float(t) for t in t_schedule]) if t_schedule is not None else None
    n_steps = len(t_schedule) if t_schedule is not None else 0
    nbytes = c_size_t(0)
    check("blk_prepare_weights", lib.blk_prepare_weights(
        byref(cfg), arr, n_layers, byref(hs) if hs is not None else None, ts, n_steps, None,
        byref(nbytes), None))
    if out is None:
        out = torch.empty(nbytes.value, dtype=torch.uint8, device="cuda")
    cap = c_size_t(out.numel())
    check("blk_prepare_weights", lib.blk_prepare_weights(
        byref(cfg), arr, n_layers, byref(hs) if hs is not None else None, ts, n_steps,
        c_void_p(out.data_ptr()), byref(cap), c_void_p(_stream(stream))))
    return out


def forward_workspace_bytes(cfg: BlkConfig, batch: int, tokens: int, prefix: int) -> int:
    lib = load()
    nbytes = c_size_t(0)
    check("blk_forward", lib.blk_forward(byref(cfg), None, 0, batch, tokens, prefix, None, None,
                                         None, 0, None, None, None, 0, None, byref(nbytes), None))
    return nbytes.value


def blk_forward(cfg: BlkConfig, packed, layer: int, x, k_prefix=None, v_prefix=None, *,
                y=None, k_new=None, v_new=None, prefix_stride=None, new_stride=None, ws=None,
                stream=None):
    """One block stage.  x: bf16 [B, T, D]; k_prefix, v_prefix: bf16 [B, P, Hkv, d]
    (or any layout with ``prefix_stride`` elements between streams).  Returns
    (y [B, T, D], k_new [B, T, Hkv, d], v_new [B, T, Hkv, d])."""
    torch = _torch()
    lib = load()
    B, T, D = x.shape
    P = 0 if k_prefix is None else k_prefix.shape[-3]
    kvrow = cfg.n_kv_heads * cfg.head_dim
    if y is None:
        y = torch.empty_like(x)
    if k_new is None:
        k_new = torch.empty(B, T, cfg.n_kv_heads, cfg.head_dim, dtype=x.dtype, device=x.device)
    if v_new is None:
        v_new = torch.empty_like(k_new)
    if prefix_stride is None:
        prefix_stride = P * kvrow
    if new_stride is None:
        new_stride = T * kvrow
    if ws is None:
        ws = torch.zeros(forward_workspace_bytes(cfg, B, T, P), dtype=torch.uint8, device=x.device)
    cap = c_size_t(ws.numel())
    check("blk_forward", lib.blk_forward(
        byref(cfg), c_void_p(packed.data_ptr()), layer, B, T, P, c_void_p(x.data_ptr()),
        c_void_p(_ptr(k_prefix)), c_void_p(_ptr(v_prefix)), prefix_stride, c_void_p(y.data_ptr()),
        c_void_p(k_new.data_ptr()), c_void_p(v_new.data_ptr()), new_stride,
        c_void_p(ws.data_ptr()), byref(cap), c_void_p(_stream(stream))))
    return y, k_new, v_new


def blk_forward_chunks(cfg: BlkConfig, packed, layer: int, x, prefix_lens, k_prefix=None,
                       v_prefix=None, *, y=None, k_new=None, v_new=None, prefix_stride=None,
                       new_stride=None, ws=None, stream=None):
    """blk_forward for chunks whose histories differ in length: stream b
    attends to the first prefix_lens[b] rows of its prefix (P = k_prefix's
    row count is the capacity) and to its own T keys; its token t is at
    position prefix_lens[b] + t.  prefix_stride=0 shares one prefix among all
    streams.  Returns (y, k_new, v_new)."""
    torch = _torch()
    lib = load()
    B, T, D = x.shape
    P = 0 if k_prefix is None else k_prefix.shape[-3]
    kvrow = cfg.n_kv_heads * cfg.head_dim
    lens = (c_int32 * max(B, 1))(*[int(v) for v in prefix_lens])
    if y is None:
        y = torch.empty_like(x)
    if k_new is None:
        k_new = torch.empty(B, T, cfg.n_kv_heads, cfg.head_dim, dtype=x.dtype, device=x.device)
    if v_new is None:
        v_new = torch.empty_like(k_new)
    if prefix_stride is None:
        prefix_stride = P * kvrow
    if new_stride is None:
        new_stride = T * kvrow
    if ws is None:
        ws = torch.zeros(forward_workspace_bytes(cfg, B, T, P), dtype=torch.uint8, device=x.device)
    cap = c_size_t(ws.numel())
    check("blk_forward_chunks", lib.blk_forward_chunks(
        byref(cfg), c_void_p(packed.data_ptr()), layer, B, T, P, lens, c_void_p(x.data_ptr()),
        c_void_p(_ptr(k_prefix)), c_void_p(_ptr(v_prefix)), prefix_stride, c_void_p(y.data_ptr()),
        c_void_p(k_new.data_ptr()), c_void_p(v_new.data_ptr()), new_stride,
        c_void_p(ws.data_ptr()), byref(cap), c_void_p(_stream(stream))))
    return y, k_new, v_new


NOALLOC_SCRATCH_BYTES = 16 << 20


def blk_forward_noalloc(cfg: BlkConfig, packed, layer: int, x, k_prefix=None, v_prefix=None, *,
                        y=None, k_new=None, v_new=None, prefix_stride=None, new_stride=None,
                        stream=None):
    """blk_forward on the library's static per-GPU scratch (no workspace
    argument, nothing allocated by the library).  Outputs not passed are
    allocated here by torch, before the call; pass y, k_new and v_new to
    allocate nothing at all."""
    torch = _torch()
    lib = load()
    B, T, D = x.shape
    P = 0 if k_prefix is None else k_prefix.shape[-3]
    kvrow = cfg.n_kv_heads * cfg.head_dim
    if y is None:
        y = torch.empty_like(x)
    if k_new is None:
        k_new = torch.empty(B, T, cfg.n_kv_heads, cfg.head_dim, dtype=x.dtype, device=x.device)
    if v_new is None:
        v_new = torch.empty_like(k_new)
    if prefix_stride is None:
        prefix_stride = P * kvrow
    if new_stride is None:
        new_stride = T * kvrow
    check("blk_forward_noalloc", lib.blk_forward_noalloc(
        byref(cfg), c_void_p(packed.data_ptr()), layer, B, T, P, c_void_p(x.data_ptr()),
        c_void_p(_ptr(k_prefix)), c_void_p(_ptr(v_prefix)), prefix_stride, c_void_p(y.data_ptr()),
        c_void_p(k_new.data_ptr()), c_void_p(v_new.data_ptr()), new_stride,
        c_void_p(_stream(stream))))
    return y, k_new, v_new


def prefill_workspace_bytes(cfg: BlkConfig, packed, n_layers: int, tokens: int) -> int:
    lib = load()
    nbytes = c_size_t(0)
    check("prefix_prefill", lib.prefix_prefill(byref(cfg), c_void_p(packed.data_ptr()), n_layers,
                                               tokens, None, None, None, None, byref(nbytes), None))
    return nbytes.value


def prefix_prefill(cfg: BlkConfig, packed, x, k_cache: list, v_cache: list, *, ws=None,
                   stream=None) -> None:
    """The prefix stage: len(k_cache) layers on the prefix tokens x (bf16
    [T, D]); layer l writes its keys and values into k_cache[l], v_cache[l]
    (bf16 [T, Hkv, d] each); the last layer computes only its keys and values."""
    torch = _torch()
    lib = load()
    L = len(k_cache)
    T = x.shape[0]
    if ws is None:
        ws = torch.zeros(prefill_workspace_bytes(cfg, packed, L, T), dtype=torch.uint8,
                         device=x.device)
    kp = (c_void_p * L)(*[t.data_ptr() for t in k_cache])
    vp = (c_void_p * L)(*[t.data_ptr() for t in v_cache])
    cap = c_size_t(ws.numel())
    check("prefix_prefill", lib.prefix_prefill(
        byref(cfg), c_void_p(packed.data_ptr()), L, T, c_void_p(x.data_ptr()), kp, vp,
        c_void_p(ws.data_ptr()), byref(cap), c_void_p(_stream(stream))))


def flow_workspace_bytes(cfg: BlkConfig, packed, n_layers: int, n_steps: int, prefix: int) -> int:
    lib = load()
    nbytes = c_size_t(0)
    check("flow_denoise", lib.flow_denoise(byref(cfg), c_void_p(packed.data_ptr()), n_layers,
                                           n_steps, prefix, None, None, None, None, None, None,
                                           byref(nbytes), None))
    return nbytes.value


def flow_denoise(cfg: BlkConfig, packed, n_steps: int, k_prefix: list, v_prefix: list, noise,
                 state, *, actions=None, ws=None, stream=None):
    """The denoise loop over len(k_prefix) layers.  k_prefix[l], v_prefix[l]: bf16
    [P, Hkv, d]; noise: float32 [N, A]; state: float32 [A].  Returns actions
    float32 [N, A].  Pass the same ``actions`` and ``ws`` tensors on every call
    to replay the cached graph."""
    torch = _torch()
    lib = load()
    L = len(k_prefix)
    P = k_prefix[0].shape[0] if L else 0
    if actions is None:
        actions = torch.empty_like(noise)
    if ws is None:
        ws = torch.zeros(flow_workspace_bytes(cfg, packed, L, n_steps, P), dtype=torch.uint8,
                         device=noise.device)
    kp = (c_void_p * L)(*[t.data_ptr() for t in k_prefix])
    vp = (c_void_p * L)(*[t.data_ptr() for t in v_prefix])
    cap = c_size_t(ws.numel())
    check("flow_denoise", lib.flow_denoise(
        byref(cfg), c_void_p(packed.data_ptr()), L, n_steps, P, kp, vp,
        c_void_p(noise.data_ptr()), c_void_p(state.data_ptr()), c_void_p(actions.data_ptr()),
        c_void_p(ws.data_ptr()), byref(cap), c_void_p(_stream(stream))))
    return actions


def blk_last_error() -> str:
    return load().blk_last_error().decode()


def blk_release() -> None:
    load().blk_release()


def blk_version() -> int:
    return load().blk_version()


EXEC_AUTO, EXEC_PER_OPERATOR, EXEC_PERSISTENT = 0, 1, 2


def blk_set_execution_mode(mode: int) -> None:
    """0 (default): automatic (at present one kernel per operator); 1: one
    kernel per operator; 2: the persistent stage kernel only."""
    check("blk_set_execution_mode", load().blk_set_execution_mode(mode))


def blk_workspace_status(ws, stream=None) -> None:
    """Wait for the stream and raise BlkError (BLK_EABORTED) if a persistent
    launch on workspace ``ws`` timed out."""
    check("blk_workspace_status", load().blk_workspace_status(c_void_p(ws.data_ptr()),
                                                              c_void_p(_stream(stream))))


def blk_set_operator_timing(enable: bool) -> None:
    """Bracket every operator of each blk_forward call with HIP events on its
    stream (or stop); either call discards what was accumulated."""
    check("blk_set_operator_timing", load().blk_set_operator_timing(1 if enable else 0))


def blk_operator_times() -> dict:
    """{operator name: (average microseconds per call, timed calls)} since
    timing was enabled, for the operators that ran."""
    n = len(OPERATORS)
    avg = (c_double * n)()
    calls = (ctypes.c_int * n)()
    check("blk_operator_times", load().blk_operator_times(avg, calls, n))
    return {OPERATORS[i]: (avg[i], calls[i]) for i in range(n) if calls[i] > 0}


def _probe_check(fn: str, rc: int) -> None:
    if rc != BLK_OK:
        raise BlkError(fn, rc, load().blk_probe_last_error().decode())


def probe_hbm_read(buf, reps: int = 10, stream=None) -> float:
    """Sustained HBM read GB/s over the device tensor ``buf`` (make it larger
    than the 256 MB last-level cache)."""
    gbs = c_double(0.0)
    _probe_check("blk_probe_hbm_read", load().blk_probe_hbm_read(
        c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(), reps, byref(gbs),
        c_void_p(_stream(stream))))
    return gbs.value


def probe_mfma_bf16(iters: int = 20000, stream=None):
    """(dense bf16 MFMA TFLOP/s, shader clock GHz under that load)."""
    tf, ghz = c_double(0.0), c_double(0.0)
    _probe_check("blk_probe_mfma_bf16", load().blk_probe_mfma_bf16(
        iters, byref(tf), byref(ghz), c_void_p(_stream(stream))))
    return tf.value, ghz.value
