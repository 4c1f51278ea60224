import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU oracle case")


def f32_tree(d):
    """Replace synth.Bf16 leaves of a dict by their exact float32 values."""
    from synth import Bf16
    return {k: (v.f32 if isinstance(v, Bf16) else v) for k, v in d.items()}


def shape_kwargs(shape):
    return dict(n_q_heads=shape.n_q_heads, n_kv_heads=shape.n_kv_heads,
                head_dim=shape.head_dim, rope_base=shape.rope_base, eps=shape.rms_eps)


def max_err_ratio(got, ref):
    """max|got - ref| / max|ref| (the parity criterion's ratio)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))
