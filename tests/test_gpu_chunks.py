"""GPU parity for blk_forward_chunks: a batch of chunks whose histories differ
in length ([PS]: AREX Feed article on PhysisServe, sections on the pipeline
per denoise step and block, where a chunk reads the cached noisy K/V of the
chunks before it, and on same-block batching across chunks).

Each stream b is checked against the oracle's block on the first
prefix_lens[b] rows of its prefix (tokens at positions prefix_lens[b] + t),
to the block tolerance max|gpu - ref| <= 1e-2 max|ref| per output tensor.
The shapes make some key slices of the shorter streams empty (the slices are
sized for the longest prefix), on both attention modes and both paths.
"""
import pytest

import oracle
import synth
from conftest import f32_tree, max_err_ratio, shape_kwargs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BLOCK_TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diffusion_transformer_block_amd as blk
    blk.blk_release()
    yield
    torch.cuda.synchronize()
    blk.blk_release()


def say(msg):
    print(f"[chunks] {msg}", flush=True)


def config_of(shape, max_pos):
    import diffusion_transformer_block_amd as blk
    return blk.make_config(shape.hidden, shape.ffn, shape.n_q_heads, shape.n_kv_heads,
                           shape.head_dim, max_pos, shape.rope_base, shape.rms_eps)


def prepared(shape, case, max_pos):
    import diffusion_transformer_block_amd as blk
    cfg = config_of(shape, max_pos)
    return cfg, blk.blk_prepare_weights(cfg, [synth.tree_to_device(case["weights"])])


def stack(case, key):
    return torch.stack([synth.to_device(st[key]) for st in case["streams"]])


def oracle_stream(shape, case, x, kp, vp):
    """The oracle's block for one stream: x [T, D] f32, kp / vp [L, Hkv, d] f32."""
    w = f32_tree(case["weights"])
    return oracle.block_forward(x, w, kp, vp, **shape_kwargs(shape))


def f(t):
    return t.float().cpu().numpy()


def check_streams(shape, case, lens, y, kn, vn, kp_of):
    """Compare every stream with the oracle on its own prefix rows."""
    for b, L in enumerate(lens):
        st = f32_tree(case["streams"][b])
        kp, vp = kp_of(b, L)
        ry, rk, rv = oracle_stream(shape, case, st["x"], kp, vp)
        ey, ek, ev = max_err_ratio(y[b], ry), max_err_ratio(kn[b], rk), max_err_ratio(vn[b], rv)
        say(f"  stream {b} (prefix {L}): y {ey:.2e}  k_new {ek:.2e}  v_new {ev:.2e}")
        assert ey <= BLOCK_TOL and ek <= BLOCK_TOL and ev <= BLOCK_TOL


CHUNK_CASES = [
    # small path, 64-row attention blocks over 5 key slices of 64: streams
    # with prefixes 0 and 37 leave slices empty
    (synth.small_shape("chunks_small_d64", hidden=256, ffn=512, n_q_heads=4, n_kv_heads=1,
                       head_dim=64, batch=4, tokens=16, prefix=300), [0, 37, 300, 128]),
    # small path at the action-expert layer shape (d = 256), two 32-token chunks
    (synth.small_shape("chunks_small_ae", hidden=1024, ffn=4096, n_q_heads=8, n_kv_heads=1,
                       head_dim=256, batch=2, tokens=32, prefix=520), [520, 100]),
    # large path, 128-row attention blocks over 4 key slices: the 123-key
    # stream leaves two slices empty
    (synth.small_shape("chunks_long_d128", hidden=512, ffn=1024, n_q_heads=16, n_kv_heads=16,
                       head_dim=128, batch=2, tokens=300, prefix=900), [900, 123]),
    # large path, d = 256 (64-row attention blocks), one stream with no history
    (synth.small_shape("chunks_large_ae", hidden=1024, ffn=4096, n_q_heads=8, n_kv_heads=1,
                       head_dim=256, batch=2, tokens=160, prefix=520), [0, 520]),
]


@pytest.mark.parametrize("shape,lens", CHUNK_CASES, ids=lambda v: getattr(v, "name", None))
def test_chunks_ragged_prefixes(shape, lens):
    import diffusion_transformer_block_amd as blk
    case = synth.block_case(shape)
    P, T = shape.prefix, shape.tokens
    cfg, packed = prepared(shape, case, P + T)
    x, kp, vp = stack(case, "x"), stack(case, "k_prefix"), stack(case, "v_prefix")
    say(f"{shape.name}: B={shape.batch} T={T} P={P} lens={lens}")
    y, kn, vn = blk.blk_forward_chunks(cfg, packed, 0, x, lens, kp, vp)
    torch.cuda.synchronize()
    kp32 = lambda b, L: (f32_tree(case["streams"][b])["k_prefix"][:L],
                         f32_tree(case["streams"][b])["v_prefix"][:L])
    check_streams(shape, case, lens, f(y), f(kn), f(vn), kp32)


def test_chunks_at_the_stream_limit():
    """16 chunks (the most one call takes) of 4 tokens, 64 rows in all, with
    history lengths from 0 to the full 200."""
    import diffusion_transformer_block_amd as blk
    shape = synth.small_shape("chunks_16x4", hidden=256, ffn=512, n_q_heads=4, n_kv_heads=1,
                              head_dim=64, batch=16, tokens=4, prefix=200)
    lens = [0, 200, 13, 64, 65, 127, 128, 1, 199, 32, 100, 150, 7, 77, 180, 50]
    case = synth.block_case(shape)
    cfg, packed = prepared(shape, case, shape.prefix + shape.tokens)
    x, kp, vp = stack(case, "x"), stack(case, "k_prefix"), stack(case, "v_prefix")
    say(f"{shape.name}: B=16 T=4 P=200 lens={lens}")
    y, kn, vn = blk.blk_forward_chunks(cfg, packed, 0, x, lens, kp, vp)
    torch.cuda.synchronize()
    kp32 = lambda b, L: (f32_tree(case["streams"][b])["k_prefix"][:L],
                         f32_tree(case["streams"][b])["v_prefix"][:L])
    check_streams(shape, case, lens, f(y), f(kn), f(vn), kp32)


def test_chunks_with_full_prefixes_equal_blk_forward():
    """Every stream at the full prefix length: the same bits as blk_forward."""
    import diffusion_transformer_block_amd as blk
    shape = CHUNK_CASES[0][0]
    case = synth.block_case(shape)
    cfg, packed = prepared(shape, case, shape.prefix + shape.tokens)
    x, kp, vp = stack(case, "x"), stack(case, "k_prefix"), stack(case, "v_prefix")
    a = blk.blk_forward(cfg, packed, 0, x, kp, vp)
    b = blk.blk_forward_chunks(cfg, packed, 0, x, [shape.prefix] * shape.batch, kp, vp)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_chunks_share_one_cache():
    """prefix_stride 0: three chunks read the first 32, 64 and 96 rows of one
    shared cache (a chunk sees the chunks before it)."""
    import diffusion_transformer_block_amd as blk
    shape = synth.small_shape("chunks_shared", hidden=256, ffn=512, n_q_heads=4, n_kv_heads=1,
                              head_dim=64, batch=3, tokens=16, prefix=96)
    case = synth.block_case(shape)
    cfg, packed = prepared(shape, case, shape.prefix + shape.tokens)
    x = stack(case, "x")
    kc = synth.to_device(case["streams"][0]["k_prefix"])   # [96, Hkv, d], shared
    vc = synth.to_device(case["streams"][0]["v_prefix"])
    lens = [32, 64, 96]
    say(f"{shape.name}: shared cache of {shape.prefix} rows, lens={lens}")
    y, kn, vn = blk.blk_forward_chunks(cfg, packed, 0, x, lens, kc, vc, prefix_stride=0)
    torch.cuda.synchronize()
    k0 = f32_tree(case["streams"][0])
    check_streams(shape, case, lens, f(y), f(kn), f(vn),
                  lambda b, L: (k0["k_prefix"][:L], k0["v_prefix"][:L]))


def test_chunk_appends_its_kv_for_the_next_interval():
    """Two pipeline intervals over one cache.  Interval 1: chunk A (history
    rows 0..63) and chunk B (history 0..31) in one call; A's K_new / V_new are
    then appended to the cache at rows 64..79.  Interval 2: chunk C reads
    rows 0..79, including what A wrote.  The oracle runs the same two
    intervals on its own: its cache takes its own K_new / V_new of A, never
    the GPU's."""
    import diffusion_transformer_block_amd as blk
    shape = synth.small_shape("chunks_interval", hidden=256, ffn=512, n_q_heads=4, n_kv_heads=1,
                              head_dim=64, batch=2, tokens=16, prefix=80)
    case = synth.block_case(shape)
    T = shape.tokens
    cfg, packed = prepared(shape, case, shape.prefix + T)
    cache_k = synth.to_device(case["streams"][0]["k_prefix"]).clone()   # [80, Hkv, d]
    cache_v = synth.to_device(case["streams"][0]["v_prefix"]).clone()
    k0 = f32_tree(case["streams"][0])
    ref_k, ref_v = k0["k_prefix"].copy(), k0["v_prefix"].copy()
    x = stack(case, "x")
    # interval 1: A = stream 0 over 64 rows, B = stream 1 over 32 rows
    y1, kn1, vn1 = blk.blk_forward_chunks(cfg, packed, 0, x, [64, 32], cache_k, cache_v,
                                          prefix_stride=0)
    torch.cuda.synchronize()
    check_streams(shape, case, [64, 32], f(y1), f(kn1), f(vn1),
                  lambda b, L: (ref_k[:L], ref_v[:L]))
    # each side's consumer appends its own K/V of A at rows 64..79
    cache_k[64:64 + T].copy_(kn1[0])
    cache_v[64:64 + T].copy_(vn1[0])
    _, ak, av = oracle_stream(shape, case, f32_tree(case["streams"][0])["x"], ref_k[:64], ref_v[:64])
    ref_k[64:64 + T], ref_v[64:64 + T] = ak, av
    # interval 2: C = stream 1's tokens again, now over 80 rows
    xc = x[1:2].contiguous()
    y2, kn2, vn2 = blk.blk_forward_chunks(cfg, packed, 0, xc, [80], cache_k, cache_v)
    torch.cuda.synchronize()
    st = f32_tree(case["streams"][1])
    ry, rk, rv = oracle_stream(shape, case, st["x"], ref_k[:80], ref_v[:80])
    ey, ek, ev = max_err_ratio(f(y2)[0], ry), max_err_ratio(f(kn2)[0], rk), max_err_ratio(f(vn2)[0], rv)
    say(f"  interval 2 (prefix 80, rows 64..79 from interval 1): y {ey:.2e}  k_new {ek:.2e}  v_new {ev:.2e}")
    assert ey <= BLOCK_TOL and ek <= BLOCK_TOL and ev <= BLOCK_TOL
