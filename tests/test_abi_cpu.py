"""The C ABI without a GPU: the library loads, exports every function the
header declares, answers size queries, and rejects bad arguments with the
documented codes before touching the device."""
import ctypes
import os
import re
import threading
from ctypes import byref, c_double, c_size_t, c_void_p

import pytest

import diffusion_transformer_block_amd as blk
from diffusion_transformer_block_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "blk.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def cfg(**kw):
    base = dict(hidden=1024, ffn=4096, n_q_heads=8, n_kv_heads=1, head_dim=256, max_pos=1024)
    base.update(kw)
    return blk.make_config(**base)


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.blk_version() == 1


def test_size_queries():
    c = cfg()
    ws = blk.forward_workspace_bytes(c, 1, 64, 520)
    assert ws > 64 * 1024 * 2 * 3
    assert ws % 256 == 0
    pb = blk.packed_bytes(c, 2)
    # two layers of 17,301,504 bf16 weights plus the RoPE table
    assert pb >= 2 * 17_301_504 * 2 + 1024 * 128 * 8
    assert blk.packed_bytes(c, 3) - pb >= 17_301_504 * 2
    # large-chunk shapes need no split-K scratch, only the activations
    c4 = cfg(hidden=1536, ffn=8960, n_q_heads=12, n_kv_heads=12, head_dim=128, max_pos=6240)
    assert blk.forward_workspace_bytes(c4, 1, 1560, 4680) >= 1560 * (3 * 1536 + 8960) * 2  # q, o, h, a


def _prep_size(lib, c, n_layers=1):
    n = c_size_t(0)
    arr = (_lib.LayerSrc * max(n_layers, 1))()
    return lib.blk_prepare_weights(byref(c), arr, n_layers, None, None, 0, None, byref(n), None), n.value


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), _lib.BLK_EUNSUPPORTED),
    (dict(n_q_heads=6, n_kv_heads=4), _lib.BLK_EUNSUPPORTED),
    (dict(hidden=1000), _lib.BLK_EUNSUPPORTED),
    (dict(ffn=4000), _lib.BLK_EUNSUPPORTED),
    (dict(hidden=0), _lib.BLK_EINVAL),
    (dict(max_pos=-1), _lib.BLK_EINVAL),
    (dict(max_pos=(1 << 20) + 1), _lib.BLK_EUNSUPPORTED),
])
def test_config_validation(lib, kw, code):
    rc, _ = _prep_size(lib, cfg(**kw))
    assert rc == code
    assert lib.blk_last_error().decode() != ""


def test_null_config_and_null_sizes(lib):
    n = c_size_t(0)
    assert lib.blk_prepare_weights(None, None, 0, None, None, 0, None, byref(n), None) == _lib.BLK_EINVAL
    c = cfg()
    assert lib.blk_prepare_weights(byref(c), None, 1, None, None, 0, None, None, None) == _lib.BLK_EINVAL
    assert lib.blk_forward(byref(c), None, 0, 1, 64, 0, None, None, None, 0, None, None, None, 0,
                           None, None, None) == _lib.BLK_EINVAL


def test_prepare_rejects_small_dst_and_null_layer_pointers(lib):
    c = cfg()
    rc, need = _prep_size(lib, c)
    assert rc == 0
    small = c_size_t(need - 1)
    arr = (_lib.LayerSrc * 1)()
    fake = c_void_p(0x1000)   # never dereferenced: validation fails first
    assert lib.blk_prepare_weights(byref(c), arr, 1, None, None, 0, fake, byref(small), None) == _lib.BLK_ESIZE
    ok = c_size_t(need)
    assert lib.blk_prepare_weights(byref(c), arr, 1, None, None, 0, fake, byref(ok), None) == _lib.BLK_EINVAL
    assert "NULL" in lib.blk_last_error().decode()


def test_prepare_flow_head_validation(lib):
    c = cfg()
    head = _lib.FlowHeadSrc(63, 32)          # all pointers NULL
    sched = (c_double * 10)(*[(10 - s) / 10 for s in range(10)])
    n = c_size_t(0)
    arr = (_lib.LayerSrc * 1)()
    assert lib.blk_prepare_weights(byref(c), arr, 1, byref(head), sched, 10, None, byref(n), None) == _lib.BLK_EINVAL
    head = _lib.FlowHeadSrc(64, 32, *([0x1000] * 11))   # 65 tokens > 64
    assert lib.blk_prepare_weights(byref(c), arr, 1, byref(head), sched, 10, None, byref(n), None) == _lib.BLK_EUNSUPPORTED
    head = _lib.FlowHeadSrc(63, 32, *([0x1000] * 11))
    assert lib.blk_prepare_weights(byref(c), arr, 1, byref(head), sched, 0, None, byref(n), None) == _lib.BLK_EUNSUPPORTED
    bad = (c_double * 10)(*([float("nan")] * 10))
    assert lib.blk_prepare_weights(byref(c), arr, 1, byref(head), bad, 10, None, byref(n), None) == _lib.BLK_EINVAL
    assert lib.blk_prepare_weights(byref(c), arr, 1, byref(head), sched, 10, None, byref(n), None) == 0
    assert n.value > blk.packed_bytes(c, 1)


def test_forward_validation_before_any_device_work(lib):
    c = cfg()
    need = blk.forward_workspace_bytes(c, 1, 64, 520)
    fake = c_void_p(0x1000)
    small = c_size_t(need - 256)
    args = lambda P, T, ws, n: (byref(c), fake, 0, 1, T, P, fake, fake, fake, 0, fake, fake, fake,
                                0, ws, byref(n), None)
    assert lib.blk_forward(*args(520, 64, fake, small)) == _lib.BLK_ESIZE
    ok = c_size_t(need)
    # packed buffer never prepared in this process
    assert lib.blk_forward(*args(520, 64, fake, ok)) == _lib.BLK_ESTATE
    # positions beyond the RoPE table
    assert lib.blk_forward(*args(1000, 64, None, ok)) == _lib.BLK_EUNSUPPORTED
    assert lib.blk_forward(*args(-1, 64, None, ok)) == _lib.BLK_EINVAL


def test_flow_denoise_unknown_packed(lib):
    c = cfg()
    n = c_size_t(0)
    assert lib.flow_denoise(byref(c), c_void_p(0x1000), 18, 10, 768, None, None, None, None, None,
                            None, byref(n), None) == _lib.BLK_ESTATE
    assert lib.flow_denoise(byref(c), None, 18, 10, 768, None, None, None, None, None, None,
                            byref(n), None) == _lib.BLK_EINVAL


def test_last_error_is_per_thread(lib):
    _prep_size(lib, cfg(head_dim=96))
    mine = lib.blk_last_error().decode()
    seen = {}

    def other():
        seen["msg"] = _lib.load().blk_last_error().decode()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert "head_dim" in mine and seen["msg"] == ""


def test_binding_raises_blk_error():
    with pytest.raises(blk.BlkError) as ei:
        blk.packed_bytes(cfg(head_dim=96), 1)
    assert ei.value.code == _lib.BLK_EUNSUPPORTED


def test_operator_timing_arguments(lib):
    assert lib.blk_set_operator_timing(2) == _lib.BLK_EINVAL
    assert lib.blk_set_operator_timing(-1) == _lib.BLK_EINVAL
    assert lib.blk_operator_times(None, None, 3) == _lib.BLK_EINVAL
    assert lib.blk_operator_times(None, None, -1) == _lib.BLK_EINVAL
    # nothing recorded: no device work, every operator reads as never run
    blk.blk_set_operator_timing(True)
    try:
        assert blk.blk_operator_times() == {}
    finally:
        blk.blk_set_operator_timing(False)
    assert len(_lib.OPERATORS) == 6


def test_bench_refuses_more_than_one_gpu():
    """The bench line is one GPU's throughput: --gpus N > 1 exits with a
    message (status 2) before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "4"],
                       capture_output=True, text=True, timeout=300, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_noalloc_rejects_a_stage_beyond_its_scratch(lib):
    """The video chunk needs far more than the static scratch: refused with
    BLK_ESIZE before any device work (no packed buffer is even looked up)."""
    c = cfg(hidden=1536, ffn=8960, n_q_heads=12, n_kv_heads=12, head_dim=128, max_pos=6240)
    assert blk.forward_workspace_bytes(c, 1, 1560, 4680) > blk.NOALLOC_SCRATCH_BYTES
    rc = lib.blk_forward_noalloc(byref(c), None, 0, 1, 1560, 4680, None, None, None, 0, None,
                                 None, None, 0, None)
    assert rc == _lib.BLK_ESIZE
    assert "scratch" in lib.blk_last_error().decode()


def test_status_and_probe_arguments(lib):
    """The workspace status query and the measurement probes reject bad
    arguments before touching the device."""
    assert lib.blk_workspace_status(None, None) == _lib.BLK_EINVAL
    g = c_double(0.0)
    assert lib.blk_probe_hbm_read(None, 1 << 30, 1, byref(g), None) == _lib.BLK_EINVAL
    assert lib.blk_probe_mfma_bf16(0, byref(g), byref(g), None) == _lib.BLK_EINVAL
    assert lib.blk_probe_mfma_bf16(10, None, byref(g), None) == _lib.BLK_EINVAL
    assert lib.blk_probe_last_error()
    hdr = open(HEADER).read()
    assert f"#define BLK_WS_ABORT_OFFSET {_lib.WS_ABORT_OFFSET}" in hdr


def test_chunks_validation_before_any_device_work(lib):
    """blk_forward_chunks checks its per-stream prefix lengths before any
    device work: NULL lengths, a length outside [0, P], and more streams than
    its kernel arguments carry are refused with the documented codes; valid
    lengths reach the packed-buffer lookup (unknown here: BLK_ESTATE)."""
    c = cfg()
    B, T, P = 4, 16, 100
    need = blk.forward_workspace_bytes(c, B, T, P)
    fake = c_void_p(0x1000)
    ok = c_size_t(need)
    Lens = ctypes.c_int32 * 17

    def call(batch, lens, ws=fake):
        return lib.blk_forward_chunks(byref(c), fake, 0, batch, T, P, lens, fake, fake, fake, 0,
                                      fake, fake, fake, T * 256, ws, byref(ok), None)

    assert call(B, None) == _lib.BLK_EINVAL
    assert "prefix_lens" in lib.blk_last_error().decode()
    assert call(B, Lens(0, 37, 101, 64)) == _lib.BLK_EINVAL
    assert call(B, Lens(0, 37, -1, 64)) == _lib.BLK_EINVAL
    assert call(17, Lens(*([5] * 17))) == _lib.BLK_EUNSUPPORTED
    assert call(B, Lens(0, 37, 100, 64)) == _lib.BLK_ESTATE
    # size query with no lengths at all
    n = c_size_t(0)
    assert lib.blk_forward_chunks(byref(c), None, 0, B, T, P, None, None, None, None, 0, None, None,
                                  None, 0, None, byref(n), None) == _lib.BLK_OK
    assert n.value == need
