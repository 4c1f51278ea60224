"""blk_forward_noalloc (the library's static per-GPU scratch, no workspace
argument) against blk_forward (a caller workspace) through the C ABI: two
calls in a row, the second on a smaller chunk, each checked to the block
tolerance against blk_forward's outputs on the same inputs."""
import numpy as np
import pytest

import synth
from conftest import max_err_ratio

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BLOCK_TOL = 1e-2


def say(msg):
    print(f"[no-alloc] {msg}", flush=True)


def _inputs(shape, tokens, prefix, seed):
    st = synth.stream_activations(shape, seed, tokens=tokens, prefix=prefix)
    dev = {k: synth.to_device(v)[None] for k, v in st.items()}
    return dev["x"], dev["k_prefix"], dev["v_prefix"]


def test_noalloc_matches_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diffusion_transformer_block_amd as blk
    shape = synth.AE_BLOCK
    cfg = blk.make_config(shape.hidden, shape.ffn, shape.n_q_heads, shape.n_kv_heads,
                          shape.head_dim, shape.prefix + shape.tokens)
    case = synth.block_case(shape)
    packed = blk.blk_prepare_weights(cfg, [synth.tree_to_device(case["weights"])])
    # the 64-token chunk over 520 cached keys, then a smaller one: 16 tokens over 100
    for tokens, prefix, seed in ((shape.tokens, shape.prefix, 5501), (16, 100, 5502)):
        say(f"AE block config: T={tokens} P={prefix}")
        x, kp, vp = _inputs(shape, tokens, prefix, seed)
        y = torch.empty_like(x)
        kn = torch.empty(1, tokens, shape.n_kv_heads, shape.head_dim, dtype=x.dtype, device="cuda")
        vn = torch.empty_like(kn)
        blk.blk_forward_noalloc(cfg, packed, 0, x, kp, vp, y=y, k_new=kn, v_new=vn)
        ry, rk, rv = blk.blk_forward(cfg, packed, 0, x, kp, vp)
        torch.cuda.synchronize()
        f = lambda t: t.float().cpu().numpy()
        errs = [max_err_ratio(f(a), f(b)) for a, b in ((y, ry), (kn, rk), (vn, rv))]
        same = all(torch.equal(a, b) for a, b in ((y, ry), (kn, rk), (vn, rv)))
        say(f"  max err ratio vs blk_forward {max(errs):.2e} (bit-identical: {same})")
        assert max(errs) <= BLOCK_TOL
        assert np.isfinite(f(y)).all()
