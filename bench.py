"""Benchmark of the block stage over cached K/V on one MI355X.

Default run (one JSON line on stdout):
  * headline: the 64-token action-expert block (hidden 1024, FFN 4096, 8 query
    heads x 256 sharing one KV head, 520 cached prefix tokens), block-stage
    microseconds with the weights cold: 16 packed-weight and prefix-KV copies
    (570 MB, over twice the 256 MB last-level cache) are used in rotation.
    One step = one block stage (the five kernels of blk_forward); the steps are
    replayed from a captured graph so host launch overhead is not timed.
  * roofline: achieved HBM GB/s of the block stage (compulsory bytes: packed
    weights, prefix K/V, x, y, K_new, V_new) against the 8 TB/s HBM3E peak.
  * loop: the full 18-layer x 10-step flow-matching loop (flow_denoise, one
    graph launch), 768 prefix tokens per layer; cold by construction (625 MB
    of weights per step).
  * large_chunk: the 1560-token video block and the 8 x 880-token batched
    block, MFMA utilisation against the 2.5 PFLOP/s bf16 dense peak.
  * cpu_baseline: the NumPy oracle on the host cores, a bounded sample of the
    headline workload.

--gpus N with N > 1 exits: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "block-stage µs + achieved HBM GB/s (64-tok) / MFMA util (large chunk)"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA


# kernels behind each operator of the 64-token stage
OP_KERNELS = {
    "qkv_rope": "sk_kernel<EpiQkvS> (RMS + fused QKV + RoPE)",
    "attention": "attn_sm_kernel<256> + attn_combine_kernel<256>",
    "o_proj": "sk_kernel<EpiResidS> (O projection + residual)",
    "gate_up": "sk_kernel<EpiGateUpS> (RMS + gate/up + SiLU*up)",
    "down": "sk_kernel<EpiResidS> (down projection + residual)",
    "stage": "stage_kernel (persistent)",
}

# HBM traffic per launch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE on this
# workload, scaled by the factor a plain copy kernel of known size gives, and
# the SHA-256 of the kernel sources when the counters were taken: a changed
# kernel reports null until it is profiled again.
TRAFFIC = {
    "qkv_rope": {"fetch": 6571292, "write": 622592, "bytes": 7193884, "sources": "047b3779ec37c6af"},
    "attention": {"fetch": 6098413, "write": 2924544, "bytes": 9022957, "sources": "047b3779ec37c6af"},
    "o_proj": {"fetch": 6389343, "write": 2364416, "bytes": 8753759, "sources": "047b3779ec37c6af"},
    "gate_up": {"fetch": 17909966, "write": 1048576, "bytes": 18958542, "sources": "047b3779ec37c6af"},
    "down": {"fetch": 11121739, "write": 2364416, "bytes": 13486155, "sources": "047b3779ec37c6af"},
}
TRAFFIC_FETCH_SCALE = 2.000   # FETCH_SIZE of a 256 MiB copy reads 128 MiB
TRAFFIC_WRITE_SCALE = 1.000   # WRITE_SIZE of the same copy reads 256 MiB
TRAFFIC_SOURCES = ("common.h", "skinny.h", "attn_small.h", "small.hip")


def sources_digest():
    """SHA-256 of the small-path kernel sources, comments and blank space
    stripped (a comment edit does not invalidate measured traffic)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "diffusion_transformer_block_amd", "csrc", f)) as fh:
            for line in fh:
                code = re.sub(r"//.*", "", line).strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def traffic_of(op):
    t = TRAFFIC.get(op)
    if not t or t["sources"] != sources_digest():
        return None
    return t["bytes"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=320, help="timed block stages (exactly)")
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--only", choices=["all", "block", "tiny", "loop", "frame", "chunks", "large",
                                       "video", "batched"],
                    default="all", help="restrict the run (for profiling)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--rotate", type=int, default=16, help="weight copies in rotation")
    ap.add_argument("--exec-mode", choices=["auto", "per_operator", "persistent"], default="auto",
                    help="blk_set_execution_mode for the small-chunk workloads")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB 4 times (the known-size "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def block_bytes(shape, P):
    """Compulsory HBM bytes of one block stage."""
    D, F, d, Hq, Hkv = shape.hidden, shape.ffn, shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    B, T = shape.batch, shape.tokens
    weights = 2 * (D * (Hq + 2 * Hkv) * d + Hq * d * D + 2 * D * F + F * D)
    kv_prefix = 2 * 2 * B * P * Hkv * d
    io = 2 * B * T * D * 2 + 2 * 2 * B * T * Hkv * d
    return weights, kv_prefix + io


def block_flops(shape, P):
    D, F, d, Hq, Hkv = shape.hidden, shape.ffn, shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    M = shape.batch * shape.tokens
    gemm = 2 * M * (D * (Hq + 2 * Hkv) * d + Hq * d * D + 2 * D * F + F * D)
    att = 2 * 2 * shape.batch * Hq * shape.tokens * (P + shape.tokens) * d
    return gemm, att


def operator_bytes(shape, P):
    """Algorithmic HBM bytes of each operator of one block stage: its weights,
    the activations it reads and the ones it writes (bf16)."""
    D, F, d, Hq, Hkv = shape.hidden, shape.ffn, shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    M = shape.batch * shape.tokens
    act = lambda n: 2 * M * n
    kv_new = 2 * 2 * M * Hkv * d
    wb, ob = block_bytes(shape, P)
    return {
        "stage": wb + ob,
        "qkv_rope": 2 * D * (Hq + 2 * Hkv) * d + act(D) + act(Hq * d) + kv_new,
        "attention": act(Hq * d) + 2 * 2 * shape.batch * P * Hkv * d + kv_new + act(Hq * d),
        "o_proj": 2 * Hq * d * D + act(Hq * d) + act(D) + act(D),
        "gate_up": 2 * 2 * D * F + act(D) + act(F),
        "down": 2 * F * D + act(F) + act(D) + act(D),
    }


def percentiles(v, qs=(10, 50, 90)):
    v = sorted(v)
    return [v[min(len(v) - 1, max(0, round(q / 100 * (len(v) - 1))))] for q in qs]


def config_of(blk, shape, max_pos=None):
    return blk.make_config(shape.hidden, shape.ffn, shape.n_q_heads, shape.n_kv_heads,
                           shape.head_dim, max_pos or (shape.prefix + shape.tokens),
                           shape.rope_base, shape.rms_eps)


def time_block(shape, steps, warmup, rotate):
    """Block-stage time with `rotate` weight / KV copies, replayed from a graph."""
    import torch
    import diffusion_transformer_block_amd as blk
    import synth
    case = synth.block_case(shape)
    cfg = config_of(blk, shape)
    w_dev = synth.tree_to_device(case["weights"])
    x = torch.stack([synth.to_device(s["x"]) for s in case["streams"]])
    kp0 = torch.stack([synth.to_device(s["k_prefix"]) for s in case["streams"]])
    vp0 = torch.stack([synth.to_device(s["v_prefix"]) for s in case["streams"]])
    packs = [blk.blk_prepare_weights(cfg, [w_dev]) for _ in range(rotate)]
    kps = [kp0.clone() for _ in range(rotate)]
    vps = [vp0.clone() for _ in range(rotate)]
    del w_dev
    B, T = shape.batch, shape.tokens
    y = torch.empty_like(x)
    kn = torch.empty(B, T, shape.n_kv_heads, shape.head_dim, dtype=torch.bfloat16, device="cuda")
    vn = torch.empty_like(kn)
    ws = torch.zeros(blk.forward_workspace_bytes(cfg, B, T, shape.prefix), dtype=torch.uint8,
                     device="cuda")

    def run(i):
        blk.blk_forward(cfg, packs[i], 0, x, kps[i], vps[i], y=y, k_new=kn, v_new=vn, ws=ws)

    # eager reference output, then the graph of one rotation (stages on
    # copies 0 .. rotate-1) and, when `steps` is not a multiple of `rotate`,
    # a graph of the remaining steps % rotate stages
    run(0)
    torch.cuda.synchronize()
    y_eager = y.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(rotate):
            run(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    def capture(n):
        g_ = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_):
            for i in range(n):
                run(i)
        return g_

    g = capture(rotate)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(y, y_eager), "graph replay differs from the eager block"
    rem = steps % rotate
    g_rem = capture(rem) if rem else None

    # warm-up: exactly `warmup` stages (eager calls, cycling the copies)
    for i in range(warmup):
        run(i % rotate)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    # timed region: exactly `steps` stages
    n_full = steps // rotate
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(n_full):
        g.replay()
    if g_rem is not None:
        g_rem.replay()
    e1.record(st)
    torch.cuda.synchronize()
    us_graph = e0.elapsed_time(e1) * 1e3 / steps
    # spread: at least 5 replays of the rotation graph, each timed
    n_pct = max(5, n_full)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_pct + 1)]
    ev[0].record(st)
    for r in range(n_pct):
        g.replay()
        ev[r + 1].record(st)
    torch.cuda.synchronize()
    per_rep = [ev[r].elapsed_time(ev[r + 1]) * 1e3 / rotate for r in range(n_pct)]
    n_rep = max(1, n_full)

    # eager (one C call per block, five launches each)
    for i in range(rotate):
        run(i)
    torch.cuda.synchronize()
    e0.record(st)
    for r in range(n_rep):
        for i in range(rotate):
            run(i)
    e1.record(st)
    torch.cuda.synchronize()
    us_eager = e0.elapsed_time(e1) * 1e3 / (n_rep * rotate)

    # warm: the graph of `rotate` stages on one copy (weights MALL-resident)
    gw = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gw):
        for _ in range(rotate):
            run(0)
    for _ in range(4):
        gw.replay()
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(n_rep):
        gw.replay()
    e1.record(st)
    torch.cuda.synchronize()
    us_warm = e0.elapsed_time(e1) * 1e3 / (n_rep * rotate)

    # per operator: HIP events the library records on this stream around each
    # operator of eager (cold, rotated) stages
    blk.blk_set_operator_timing(True)
    try:
        for r in range(n_rep):
            for i in range(rotate):
                run(i)
        ops = blk.blk_operator_times()
    finally:
        blk.blk_set_operator_timing(False)
    torch.cuda.synchronize()
    del g, g_rem, gw, packs, kps, vps
    torch.cuda.empty_cache()
    return {"us": us_graph, "us_eager": us_eager, "us_warm": us_warm,
            "us_p10_p50_p90": percentiles(per_rep), "pct_replays": n_pct, "timed_steps": steps,
            "ops": ops}


def time_loop(warmup, reps=20):
    import torch
    import diffusion_transformer_block_amd as blk
    import synth
    flow = synth.FLOW
    case = synth.flow_case(flow)
    fb = flow.block
    cfg = config_of(blk, fb, fb.prefix + flow.n_actions + 1)
    layers = [synth.tree_to_device(l) for l in case["layers"]]
    head = synth.tree_to_device(case["head"])
    head["n_actions"] = flow.n_actions
    packed = blk.blk_prepare_weights(cfg, layers, head, list(case["schedule"]))
    kp = [l["k_prefix"] for l in layers]
    vp = [l["v_prefix"] for l in layers]
    for l in layers:
        for k in list(l):
            if k not in ("k_prefix", "v_prefix"):
                del l[k]
    ws = torch.zeros(blk.flow_workspace_bytes(cfg, packed, flow.n_layers, flow.n_steps,
                                              fb.prefix), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(head["noise"])
    call = lambda: blk.flow_denoise(cfg, packed, flow.n_steps, kp, vp, head["noise"],
                                    head["state"], actions=out, ws=ws)
    for _ in range(max(2, warmup // 8)):
        call()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        call()
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    w_bytes, _ = block_bytes(fb, fb.prefix)
    D, A = fb.hidden, flow.action_dim
    head_bytes = 2 * D * D + 4 * (A * D * 3 + 3 * D)     # W3 bf16, W_fused/Ws/W_out f32, biases
    kv_bytes = 2 * 2 * fb.prefix * fb.n_kv_heads * fb.head_dim
    step_bytes = flow.n_layers * (w_bytes + kv_bytes) + head_bytes
    gbs = flow.n_steps * step_bytes / (ms * 1e-3) / 1e9
    del packed, ws
    torch.cuda.empty_cache()
    return {"workload": flow.name, "layers": flow.n_layers, "steps": flow.n_steps,
            "prefix": fb.prefix, "ms_per_loop": round(ms, 4),
            "us_per_layer_step": round(ms * 1e3 / (flow.n_layers * flow.n_steps), 3),
            "achieved_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "timed_loops": reps}


def time_frame(reps=10):
    """The prefix stage (18 layers over the 768 prefix tokens, last layer K/V
    only) beside the denoise loop on a second stream: the prefix stage writes
    one set of per-layer caches while the loop reads the other (the pages'
    two-stream schedule).  Times each alone, one after the other on one stream,
    and both at once; then the loop with 16 Euler steps (16 action-expert
    calls per prefix frame) beside the prefix stage."""
    import torch
    import diffusion_transformer_block_amd as blk
    import synth
    flow = synth.FLOW
    fb = flow.block
    T, L = fb.prefix, flow.n_layers
    cfg = config_of(blk, fb, fb.prefix + flow.n_actions + 1)
    case = synth.flow_case(flow)
    head = synth.tree_to_device(case["head"])
    head["n_actions"] = flow.n_actions
    loop_layers = [synth.tree_to_device(l) for l in case["layers"]]
    packed10 = blk.blk_prepare_weights(cfg, loop_layers, head, list(case["schedule"]))
    sched16 = [(16 - s_) / 16 for s_ in range(16)]
    packed16 = blk.blk_prepare_weights(cfg, loop_layers, head, sched16)
    del loop_layers
    pre_layers = [synth.tree_to_device(synth.layer_weights(fb, 7700 + l)) for l in range(L)]
    packed_pre = blk.blk_prepare_weights(cfg, pre_layers, None, None)
    del pre_layers
    x = synth.to_device(synth.stream_activations(fb, 7700, tokens=T, prefix=0)["x"])
    kv = lambda: [torch.empty(T, fb.n_kv_heads, fb.head_dim, dtype=torch.bfloat16, device="cuda")
                  for _ in range(L)]
    kc_a, vc_a, kc_b, vc_b = kv(), kv(), kv(), kv()
    pws = torch.zeros(blk.prefill_workspace_bytes(cfg, packed_pre, L, T), dtype=torch.uint8, device="cuda")
    lws10 = torch.zeros(blk.flow_workspace_bytes(cfg, packed10, L, 10, T), dtype=torch.uint8, device="cuda")
    lws16 = torch.zeros(blk.flow_workspace_bytes(cfg, packed16, L, 16, T), dtype=torch.uint8, device="cuda")
    out10, out16 = torch.empty_like(head["noise"]), torch.empty_like(head["noise"])
    s_pre = torch.cuda.Stream()
    # the caches the loop reads: one prefix pass
    blk.prefix_prefill(cfg, packed_pre, x, kc_a, vc_a, ws=pws)
    torch.cuda.synchronize()
    # the prefix stage as a graph (the loop captures its own on first use)
    g_pre = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s_pre):
        blk.prefix_prefill(cfg, packed_pre, x, kc_b, vc_b, ws=pws, stream=s_pre)
        torch.cuda.synchronize()
        with torch.cuda.graph(g_pre, stream=s_pre):
            blk.prefix_prefill(cfg, packed_pre, x, kc_b, vc_b, ws=pws, stream=s_pre)
    loop10 = lambda st: blk.flow_denoise(cfg, packed10, 10, kc_a, vc_a, head["noise"], head["state"],
                                         actions=out10, ws=lws10, stream=st)
    loop16 = lambda st: blk.flow_denoise(cfg, packed16, 16, kc_a, vc_a, head["noise"], head["state"],
                                         actions=out16, ws=lws16, stream=st)
    for _ in range(2):
        loop10(None)
        loop16(None)
        g_pre.replay()
    torch.cuda.synchronize()

    main = torch.cuda.current_stream()

    def timed(body):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(main)
        for _ in range(reps):
            body()
        e1.record(main)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def concurrent(loop):
        # the loop on the launch stream, the prefix stage on a second stream
        # that starts with it and that the launch stream waits for
        def body():
            s_pre.wait_stream(main)
            with torch.cuda.stream(s_pre):
                g_pre.replay()
            loop(main)
            main.wait_stream(s_pre)
        return body

    r = {"prefill_ms": timed(lambda: g_pre.replay()), "loop10_ms": timed(lambda: loop10(main)),
         "loop16_ms": timed(lambda: loop16(main)),
         "sequential_ms": timed(lambda: (g_pre.replay(), loop10(main))),
         "concurrent_ms": timed(concurrent(loop10)),
         "sequential16_ms": timed(lambda: (g_pre.replay(), loop16(main))),
         "concurrent16_ms": timed(concurrent(loop16))}
    out = {"workload": "prefix 18 layers x 768 tokens (last layer K/V only) beside flow_18x10",
           "reps": reps}
    out.update({k: round(v, 4) for k, v in r.items()})
    out["overlap_saved_ms"] = round(r["sequential_ms"] - r["concurrent_ms"], 4)
    # the frame at 16 calls: whichever schedule ran it faster (the prefix
    # stage's GEMMs beside a long chain of small loop kernels can cost the
    # loop more than the overlap gains)
    two = r["concurrent16_ms"] <= r["sequential16_ms"]
    frame16 = r["concurrent16_ms"] if two else r["sequential16_ms"]
    out["frame16_schedule"] = "two streams" if two else "one stream"
    out["ae_calls_per_s_16_per_frame"] = round(16 / (frame16 * 1e-3), 1)
    out["frames_per_s_16"] = round(1 / (frame16 * 1e-3), 1)
    del packed10, packed16, packed_pre, pws, lws10, lws16
    torch.cuda.empty_cache()
    return out


def time_chunks(reps=20):
    """A same-block batch of chunks at different points of one history
    (blk_forward_chunks: one shared cache, a prefix length per chunk) against
    the same chunks as separate blk_forward calls, each variant replayed from
    a captured graph with the weights resident: the batch reads the weights
    once and launches each operator once for all its chunks."""
    import dataclasses
    import torch
    import diffusion_transformer_block_amd as blk
    import synth
    cases = [("ae_4x16tok_chunks", dataclasses.replace(synth.AE_BLOCK, tokens=16), [520, 536, 552, 568]),
             ("video_2x1560tok_chunks", synth.VIDEO_DIT, [4680, 6240])]
    out = []
    for name, shape, lens in cases:
        B, T, P = len(lens), shape.tokens, max(lens)
        cfg = config_of(blk, shape, P + T)
        packed = blk.blk_prepare_weights(cfg, [synth.tree_to_device(synth.layer_weights(shape, 8800))])
        cache = synth.stream_activations(shape, 8800, tokens=T, prefix=P)
        kc, vc = synth.to_device(cache["k_prefix"]), synth.to_device(cache["v_prefix"])
        x = torch.stack([synth.to_device(synth.stream_activations(shape, 8801 + b, tokens=T, prefix=0)["x"])
                         for b in range(B)])
        y = torch.empty_like(x)
        kn = torch.empty(B, T, shape.n_kv_heads, shape.head_dim, dtype=torch.bfloat16, device="cuda")
        vn = torch.empty_like(kn)
        ws = torch.zeros(blk.forward_workspace_bytes(cfg, B, T, P), dtype=torch.uint8, device="cuda")

        def batched():
            blk.blk_forward_chunks(cfg, packed, 0, x, lens, kc, vc, prefix_stride=0, y=y, k_new=kn,
                                   v_new=vn, ws=ws)

        def separate():
            for b, L in enumerate(lens):
                blk.blk_forward(cfg, packed, 0, x[b:b + 1], kc[:L], vc[:L], y=y[b:b + 1],
                                k_new=kn[b:b + 1], v_new=vn[b:b + 1], ws=ws)

        res = {"workload": name, "chunks": B, "tokens": T, "prefix_lens": lens}
        for key, body in (("batched_us", batched), ("separate_us", separate)):
            body()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                body()
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            st = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(reps):
                g.replay()
            e1.record(st)
            torch.cuda.synchronize()
            res[key] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
            del g
        res["saved_frac"] = round(1 - res["batched_us"] / res["separate_us"], 4)
        out.append(res)
        del packed, kc, vc, x, y, kn, vn, ws
        torch.cuda.empty_cache()
    return out


def time_large(shape, reps):
    import torch
    import diffusion_transformer_block_amd as blk
    import synth
    case = synth.block_case(shape)
    cfg = config_of(blk, shape)
    packed = blk.blk_prepare_weights(cfg, [synth.tree_to_device(case["weights"])])
    x = torch.stack([synth.to_device(s["x"]) for s in case["streams"]])
    kp = torch.stack([synth.to_device(s["k_prefix"]) for s in case["streams"]])
    vp = torch.stack([synth.to_device(s["v_prefix"]) for s in case["streams"]])
    B, T = shape.batch, shape.tokens
    y = torch.empty_like(x)
    kn = torch.empty(B, T, shape.n_kv_heads, shape.head_dim, dtype=torch.bfloat16, device="cuda")
    vn = torch.empty_like(kn)
    ws = torch.zeros(blk.forward_workspace_bytes(cfg, B, T, shape.prefix), dtype=torch.uint8,
                     device="cuda")
    run = lambda: blk.blk_forward(cfg, packed, 0, x, kp, vp, y=y, k_new=kn, v_new=vn, ws=ws)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        run()
    e1.record(st)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    gemm, att = block_flops(shape, shape.prefix)
    tflops = (gemm + att) / (us * 1e-6) / 1e12
    del packed, x, kp, vp, ws
    torch.cuda.empty_cache()
    return {"workload": shape.name, "us_per_block": round(us, 2),
            "gemm_gflop": round(gemm / 1e9, 2), "attn_gflop": round(att / 1e9, 2),
            "achieved_TFLOPs": round(tflops, 1), "mfma_util": round(tflops / BF16_PEAK_TFLOPS, 4),
            "timed_blocks": reps}


def cpu_model():
    """The host CPU's model name (what lscpu prints as 'Model name')."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(budget_s=4.0, runs=3):
    """The oracle, as it stands, timed on the host on the headline workload:
    `runs` runs of about `budget_s` seconds each, median per-stage time."""
    import numpy as np
    import oracle
    import synth
    shape = synth.AE_BLOCK
    case = synth.block_case(shape)
    w = {k: (v.f32 if isinstance(v, synth.Bf16) else v) for k, v in case["weights"].items()}
    st = case["streams"][0]
    kw = dict(n_q_heads=shape.n_q_heads, n_kv_heads=shape.n_kv_heads, head_dim=shape.head_dim,
              rope_base=shape.rope_base, eps=shape.rms_eps)
    x, kp, vp = st["x"].f32, st["k_prefix"].f32, st["v_prefix"].f32
    oracle.block_forward(x, w, kp, vp, **kw)    # warm
    per_run, counts = [], []
    for _ in range(runs):
        n = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            oracle.block_forward(x, w, kp, vp, **kw)
            n += 1
        per_run.append((time.perf_counter() - t0) / n * 1e6)
        counts.append(n)
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    med = sorted(per_run)[len(per_run) // 2]
    return {"value": round(med, 1), "unit": "us", "cores": int(threads), "kind": "oracle",
            "sample": f"{runs} runs of about {budget_s:.0f} s each ({', '.join(map(str, counts))} "
                      f"block stages of the 64-token AE block, NumPy float32); median per stage",
            "runs_us": [round(v, 1) for v in per_run], "statistic": f"median of {runs}",
            "cpu_model": cpu_model(), "host_cpus_visible": len(os.sched_getaffinity(0))}


def measured_peaks():
    """The chip's sustained HBM read bandwidth, dense bf16 MFMA throughput and
    shader clock under that load, from the library's probes."""
    import torch
    import diffusion_transformer_block_amd as blk
    buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")   # 2 GiB: 8x the last-level cache
    hbm = blk.probe_hbm_read(buf, reps=5)
    del buf
    torch.cuda.empty_cache()
    tf, ghz = blk.probe_mfma_bf16(20000)
    return {"hbm_read_GBs": {"nominal": HBM_PEAK_GBS, "measured": round(hbm, 1),
                             "probe": "blk_probe_hbm_read: 5 passes of 16-byte non-temporal loads over 2 GiB"},
            "bf16_mfma_TFLOPs": {"nominal": BF16_PEAK_TFLOPS, "measured": round(tf, 1),
                                 "probe": "blk_probe_mfma_bf16: 4 chains of 32x32x16 MFMAs per wave, 2 waves per SIMD"},
            "shader_clock_GHz_under_mfma": round(ghz, 3),
            "nominal_clock_GHz": 2.4}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py: this build runs on one GPU; --gpus {max(args.gpus, world)} is not "
              "supported (the stage shards by pipeline stage and stream, see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    import diffusion_transformer_block_amd as blk
    blk.blk_set_execution_mode({"auto": blk.EXEC_AUTO, "per_operator": blk.EXEC_PER_OPERATOR,
                                "persistent": blk.EXEC_PERSISTENT}[args.exec_mode])
    if args.calib_copy > 0:
        n = args.calib_copy * (1 << 20) // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calib_copy} MiB read + {args.calib_copy} MiB written, 4 times")
        del src, dst
    rotate = max(1, args.rotate)
    steps = max(1, args.steps)
    shape = synth.AE_BLOCK
    line = {"metric": METRIC}
    if args.only in ("all", "block"):
        log("measured peaks (probes)")
        line["peaks"] = measured_peaks()
        log(f"  {line['peaks']}")
    if args.only in ("all", "block"):
        log(f"block {shape.name}: {steps} timed stages, {rotate} weight copies")
        r = time_block(shape, steps, args.warmup, rotate)
        wb, ob = block_bytes(shape, shape.prefix)
        gbs = (wb + ob) / (r["us"] * 1e-6) / 1e9
        opb = operator_bytes(shape, shape.prefix)
        operators = []
        for name, (us, calls) in r["ops"].items():
            ach = opb[name] / (us * 1e-6) / 1e9
            operators.append({"operator": name, "kernels": OP_KERNELS[name], "us": round(us, 3),
                              "calls": calls, "algorithmic_bytes": opb[name],
                              "achieved_GBs": round(ach, 1), "frac": round(ach / HBM_PEAK_GBS, 4),
                              "traffic": traffic_of(name)})
        dom = max(operators, key=lambda o: o["us"])
        op_traffic = [o["traffic"] for o in operators]
        stage_traffic = sum(op_traffic) if op_traffic and all(t is not None for t in op_traffic) else None
        line.update({
            "value": round(r["us"], 3), "unit": "us", "n_gpus": 1, "steps": r["timed_steps"],
            "warmup": args.warmup, "ms_per_step": round(r["us"] / 1e3, 6),
            "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) activations / K/V, N(0,0.02^2) weights)",
            "config": {"workload": shape.name, "hidden": shape.hidden, "ffn": shape.ffn,
                       "q_heads": shape.n_q_heads, "kv_heads": shape.n_kv_heads,
                       "head_dim": shape.head_dim, "tokens": shape.tokens,
                       "prefix": shape.prefix, "weight_copies": rotate,
                       "parallelism": "single GPU"},
            "eager_us": round(r["us_eager"], 3),
            "warm_us": round(r["us_warm"], 3),
            "us_p10_p50_p90": [round(v, 3) for v in r["us_p10_p50_p90"]],
            "pct_replays": r["pct_replays"],
            "roofline": {"bound": "hbm",
                         "kernel": "the 64-token block stage: " + " -> ".join(
                             o["kernels"] for o in operators),
                         "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": wb + ob,
                         "us_per_launch": round(r["us"], 3),
                         "timing": "HIP events on the launch stream around graph replays of whole stages",
                         "traffic": stage_traffic,
                         "dominant_operator": {"operator": dom["operator"], "us": dom["us"],
                                               "frac": dom["frac"]}},
            "stage_roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                               "algorithmic_bytes": wb + ob,
                               "roofline_us": round((wb + ob) / (HBM_PEAK_GBS * 1e3), 3)},
            "operators": operators,
        })
        log(f"  {r['us']:.2f} us/stage graph, {r['us_eager']:.2f} us eager, "
            f"{r['us_warm']:.2f} us warm, {gbs:.0f} GB/s")
        for o in operators:
            log(f"    {o['operator']:9s} {o['us']:7.2f} us  {o['achieved_GBs']:7.1f} GB/s")
    if args.only in ("all", "tiny"):
        tiny = synth.TINY
        log(f"block {tiny.name}: {steps} timed stages, {rotate} weight copies")
        r = time_block(tiny, steps, args.warmup, rotate)
        wb, ob = block_bytes(tiny, tiny.prefix)
        gbs = (wb + ob) / (r["us"] * 1e-6) / 1e9
        line["tiny_block"] = {
            "workload": tiny.name, "us": round(r["us"], 3), "us_eager": round(r["us_eager"], 3),
            "us_p10_p50_p90": [round(v, 3) for v in r["us_p10_p50_p90"]],
            "algorithmic_bytes": wb + ob, "achieved_GBs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "timed_steps": r["timed_steps"],
            "operators_us": {k: round(v[0], 3) for k, v in r["ops"].items()}}
        log(f"  {line['tiny_block']}")
    if args.only in ("all", "loop"):
        log("loop flow_18x10")
        line["loop"] = time_loop(args.warmup)
        log(f"  {line['loop']}")
    if args.only in ("all", "frame"):
        log("prefix stage beside the loop (two streams)")
        line["frame"] = time_frame()
        log(f"  {line['frame']}")
    if args.only in ("all", "chunks"):
        log("same-block batch of chunks with their own history lengths")
        line["chunks"] = time_chunks()
        log(f"  {line['chunks']}")
    if args.only in ("all", "large", "video", "batched"):
        large = []
        if args.only in ("all", "large", "video"):
            log("large chunk video_dit_1560tok")
            large.append(time_large(synth.VIDEO_DIT, 20))
            log(f"  {large[-1]}")
        if args.only in ("all", "large", "batched"):
            log("large chunk batched_8x880tok")
            large.append(time_large(synth.BATCHED, 5))
            log(f"  {large[-1]}")
        line["large_chunk"] = large
    if args.only in ("all", "block") and not args.no_cpu:
        log("cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline()
    torch.cuda.synchronize()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
