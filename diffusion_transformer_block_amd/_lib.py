"""ctypes declarations of libblk.so's C ABI (include/blk.h), one-to-one."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libblk.so")

BLK_OK = 0
BLK_EINVAL = -1
BLK_EUNSUPPORTED = -2
BLK_ESIZE = -3
BLK_ESTATE = -4
BLK_EHIP = -5
BLK_EABORTED = -6
ERROR_NAMES = {BLK_EINVAL: "BLK_EINVAL", BLK_EUNSUPPORTED: "BLK_EUNSUPPORTED",
               BLK_ESIZE: "BLK_ESIZE", BLK_ESTATE: "BLK_ESTATE", BLK_EHIP: "BLK_EHIP",
               BLK_EABORTED: "BLK_EABORTED"}
WS_ABORT_OFFSET = 110600   # BLK_WS_ABORT_OFFSET

# every function include/blk.h declares
EXPORTS = ("blk_prepare_weights", "blk_forward", "blk_forward_chunks", "blk_forward_noalloc",
           "prefix_prefill",
           "flow_denoise", "blk_last_error",
           "blk_release", "blk_version", "blk_set_execution_mode", "blk_set_operator_timing",
           "blk_operator_times", "blk_workspace_status", "blk_probe_hbm_read", "blk_probe_mfma_bf16", "blk_probe_last_error")

# operator indices of blk_operator_times (BLK_OP_* in include/blk.h)
OPERATORS = ("qkv_rope", "attention", "o_proj", "gate_up", "down", "stage")


class BlkConfig(ctypes.Structure):
    _fields_ = [("hidden", c_int32), ("ffn", c_int32), ("n_q_heads", c_int32),
                ("n_kv_heads", c_int32), ("head_dim", c_int32), ("max_pos", c_int32),
                ("rope_base", c_float), ("rms_eps", c_float)]


LAYER_FIELDS = ("g_attn", "w_q", "w_k", "w_v", "w_o", "g_ffn", "w_gate", "w_up", "w_down")
HEAD_FIELDS = ("w1", "b1", "w2", "b2", "w3", "b3", "ws", "bs", "g_f", "w_out", "b_out")


class LayerSrc(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in LAYER_FIELDS]


class FlowHeadSrc(ctypes.Structure):
    _fields_ = [("n_actions", c_int32), ("action_dim", c_int32)] + [(n, c_void_p) for n in HEAD_FIELDS]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libblk.so and declare its signatures.  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m diffusion_transformer_block_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(path)
    lib.blk_prepare_weights.argtypes = [POINTER(BlkConfig), POINTER(LayerSrc), c_int,
                                        POINTER(FlowHeadSrc), POINTER(c_double), c_int, c_void_p,
                                        POINTER(c_size_t), c_void_p]
    lib.blk_prepare_weights.restype = c_int
    lib.blk_forward.argtypes = [POINTER(BlkConfig), c_void_p, c_int, c_int, c_int, c_int,
                                c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p,
                                c_void_p, c_int64, c_void_p, POINTER(c_size_t), c_void_p]
    lib.blk_forward.restype = c_int
    lib.blk_forward_chunks.argtypes = [POINTER(BlkConfig), c_void_p, c_int, c_int, c_int, c_int,
                                       POINTER(c_int32), c_void_p, c_void_p, c_void_p, c_int64,
                                       c_void_p, c_void_p, c_void_p, c_int64, c_void_p,
                                       POINTER(c_size_t), c_void_p]
    lib.blk_forward_chunks.restype = c_int
    lib.blk_forward_noalloc.argtypes = [POINTER(BlkConfig), c_void_p, c_int, c_int, c_int, c_int,
                                        c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p,
                                        c_void_p, c_int64, c_void_p]
    lib.blk_forward_noalloc.restype = c_int
    lib.prefix_prefill.argtypes = [POINTER(BlkConfig), c_void_p, c_int, c_int, c_void_p,
                                   POINTER(c_void_p), POINTER(c_void_p), c_void_p, POINTER(c_size_t),
                                   c_void_p]
    lib.prefix_prefill.restype = c_int
    lib.flow_denoise.argtypes = [POINTER(BlkConfig), c_void_p, c_int, c_int, c_int,
                                 POINTER(c_void_p), POINTER(c_void_p), c_void_p, c_void_p,
                                 c_void_p, c_void_p, POINTER(c_size_t), c_void_p]
    lib.flow_denoise.restype = c_int
    lib.blk_last_error.argtypes = []
    lib.blk_last_error.restype = ctypes.c_char_p
    lib.blk_release.argtypes = []
    lib.blk_release.restype = None
    lib.blk_version.argtypes = []
    lib.blk_version.restype = c_int
    lib.blk_set_execution_mode.argtypes = [c_int]
    lib.blk_set_execution_mode.restype = c_int
    lib.blk_set_operator_timing.argtypes = [c_int]
    lib.blk_set_operator_timing.restype = c_int
    lib.blk_operator_times.argtypes = [POINTER(c_double), POINTER(c_int), c_int]
    lib.blk_operator_times.restype = c_int
    lib.blk_workspace_status.argtypes = [c_void_p, c_void_p]
    lib.blk_workspace_status.restype = c_int
    lib.blk_probe_hbm_read.argtypes = [c_void_p, c_size_t, c_int, POINTER(c_double), c_void_p]
    lib.blk_probe_hbm_read.restype = c_int
    lib.blk_probe_mfma_bf16.argtypes = [c_int, POINTER(c_double), POINTER(c_double), c_void_p]
    lib.blk_probe_mfma_bf16.restype = c_int
    lib.blk_probe_last_error.argtypes = []
    lib.blk_probe_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


class BlkError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} -> {ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


def check(fn: str, rc: int) -> None:
    if rc != BLK_OK:
        raise BlkError(fn, rc, load().blk_last_error().decode())
