"""Benchmark: jagged HSTU layer forward on one MI355X.

A step is one forward pass of a 24-layer HSTU stack (independent random weights per
layer, Y of layer l is X of layer l+1) over the 8 x 8192-token batch, d = 1024, 8 heads
of 128, causal mask with positional + log-time relative bias: every kernel of the hot
path (jagged schedule, f1 + SiLU, pointwise attention, LayerNorm + gate, f2) runs once
per layer.  Inputs and weights are resident in HBM before the timed region.

Prints one JSON line on stdout; progress goes to stderr.

Besides the step, the line carries separate measurements of Stochastic Length, M-FALCON
serving, the attention gradients (hstu_attn_bwd) and one layer's backward (hstu_layer_bwd).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers 24] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HSTU jagged attn+layer fwd TFLOP/s (bf16) and % MFMA peak at N=8192, 1 GPU"
PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "attention_traffic.json")
ATTN_SRC = os.path.join(ROOT, "hstu_pointwise_attention_jagged_amd", "csrc", "attention.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def useful_flops(lengths, d, H, dqk, dv):
    """MFMA work of one layer over unpadded sequences (elementwise work not counted).

    f1: 2 T d 2H(dqk+dv); attention: H (dqk+dv) n (n+1) per sequence (QK^T and AV over
    the causal triangle, diagonal included); f2: 2 T H dv d.
    """
    T = int(sum(lengths))
    f1 = 2 * T * d * 2 * H * (dqk + dv)
    att = sum(H * (dqk + dv) * int(n) * (int(n) + 1) for n in lengths)
    f2 = 2 * T * H * dv * d
    return f1, att, f2


def file_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_record():
    """HBM bytes per attention launch from committed counter runs, if still current."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("attention_hip_sha256") != file_sha(ATTN_SRC):
        return None  # kernel changed since the counters were taken
    return rec.get("bytes_per_launch")


def _counter_kib(db, kernel_substr):
    """Per-dispatch counter values (KiB) of the kernels whose name contains kernel_substr."""
    import sqlite3
    con = sqlite3.connect(db)
    vals = [v for name, v in con.execute("select name, counter_value from pmc_events")
            if kernel_substr in name]
    con.close()
    return vals


def write_traffic_record(d, copy_bytes):
    """HBM bytes per attention launch, from FETCH_SIZE / WRITE_SIZE scaled by a plain copy."""
    att_fetch = _counter_kib(os.path.join(d, "pmc_fetch", "pmc_results.db"), "attn_kernel")
    att_write = _counter_kib(os.path.join(d, "pmc_write", "pmc_results.db"), "attn_kernel")
    cp_fetch = _counter_kib(os.path.join(d, "pmc_cfetch", "pmc_results.db"), "copyBuffer")
    cp_write = _counter_kib(os.path.join(d, "pmc_cwrite", "pmc_results.db"), "copyBuffer")
    fetch_scale = copy_bytes / (1024.0 * sum(cp_fetch) / len(cp_fetch))
    write_scale = copy_bytes / (1024.0 * sum(cp_write) / len(cp_write))
    fetch_b = 1024.0 * sum(att_fetch) / len(att_fetch) * fetch_scale
    write_b = 1024.0 * sum(att_write) / len(att_write) * write_scale
    rec = {
        "kernel": "attn_kernel (8 x 8192 tokens, 8 heads x 128, causal, rab pos+time)",
        "attention_hip_sha256": file_sha(ATTN_SRC),
        "fetch_kib_per_launch": sum(att_fetch) / len(att_fetch),
        "write_kib_per_launch": sum(att_write) / len(att_write),
        "copy_bytes": copy_bytes,
        "copy_fetch_kib": sum(cp_fetch) / len(cp_fetch),
        "copy_write_kib": sum(cp_write) / len(cp_write),
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "fetch_bytes_per_launch": fetch_b,
        "write_bytes_per_launch": write_b,
        "bytes_per_launch": fetch_b + write_b,
    }
    with open(TRAFFIC_RECORD, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    log(f"wrote {TRAFFIC_RECORD}: {rec['bytes_per_launch'] / 1e6:.1f} MB per launch")


def cpu_baseline(w, layers, n_seq=2):
    """fp64 oracle on the first n_seq 8192-token sequences of the same batch, one layer."""
    import numpy as np
    from oracle import hstu_ref

    d = w.dims
    cores = min(os.cpu_count() or 1, 16)
    s0, s1 = int(w.seq.offsets[0]), int(w.seq.offsets[n_seq])
    x = w.x[s0:s1]
    off = (w.seq.offsets[: n_seq + 1] - s0).astype(np.int32)
    ts = w.seq.timestamps[s0:s1]
    t0 = time.perf_counter()
    hstu_ref.layer_fwd(x, w.weights, off, ts, d.num_heads, d.dqk, d.dv, d.ln_eps, workers=cores)
    dt = time.perf_counter() - t0
    lengths = [int(n) for n in np.diff(off)]
    f1, att, f2 = useful_flops(lengths, d.d_model, d.num_heads, d.dqk, d.dv)
    return {"value": round((f1 + att + f2) / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"one layer (not the {layers}-layer stack) on {n_seq} of the 8 sequences "
                      f"({sum(lengths)} tokens), fp64 NumPy, {dt:.1f} s",
            "seconds": round(dt, 3)}


def sl_measure(torch, np, ops, dev, wl, reps=20):
    """Stochastic Length on the 128-user raw batch (d = 512 rows gathered), timed alone.

    Algorithmic bytes: the priorities once (4 B per raw token) and, per kept token, its
    row read and written (2 x 2 d B), its timestamp read and written and its index
    written (12 B).  Offsets and per-user draws are negligible.
    """
    w = wl.config(3)
    r = w.raw
    raw = dev.jagged_of(r.seq)
    u = torch.from_numpy(r.u_keep.astype(np.float64)).cuda()
    keys = torch.from_numpy(r.keys.view(np.int32)).cuda()
    x = dev.bf16_tensor(r.x)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        _, new_off, _, _ = ops.hstu_stochastic_length(raw, u, keys, x=x, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        ops.hstu_stochastic_length(raw, u, keys, x=x, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    T_raw, T_new, dm = r.seq.total, int(new_off[-1].item()), w.dims.d_model
    alg = 4 * T_raw + T_new * (4 * dm + 12)
    return {"workload": f"stochastic length on {r.seq.batch} users, raw lengths log-uniform on "
                        f"[256, 4096], N=4096, alpha=1.6, d={dm} rows gathered",
            "raw_tokens": T_raw, "kept_tokens": T_new, "ms": round(ms, 4),
            "raw_tokens_per_s": round(T_raw / (ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(alg / (ms * 1e-3) / 1e9, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes": alg}}


def bwd_measure(torch, np, ops, dev, wl, reps=10):
    """Attention gradients (hstu_attn_bwd: dQ, dK, dV) on the 8 x 8192-token batch, 8 heads
    of 128, causal with positional + log-time bias.  Q, K, V are fp16 N(0.2, 0.6^2), dO
    fp32 N(0, 1), drawn on the device from a fixed seed.  Algorithmic FLOPs: five
    products per allowed pair and head (S, dA, dQ, dK, dV), 2 dh each, i.e.
    10 dh H n (n + 1) / 2 per sequence; the kernels recompute S and dA once more (one
    pass per side), which is not counted."""
    w = wl.config(2)
    d = w.dims
    H, dh = d.num_heads, d.dqk
    T = w.seq.total
    seq = dev.jagged_of(w.seq)
    dims = dev.dims_of(d)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3003)
    qkv = (0.2 + 0.6 * torch.randn((T, 3 * H * dh), generator=gen, device="cuda")).half()
    g = torch.randn((T, H * dh), generator=gen, device="cuda")
    rp, rt = dev.f32_tensor(w.weights.rab_pos), dev.f32_tensor(w.weights.rab_time)
    hq = H * dh
    stream = torch.cuda.current_stream()
    ws = torch.empty(int(ops.hstu_attn_bwd_workspace_bytes(dims, seq)), dtype=torch.uint8,
                     device="cuda")

    def run():
        return ops.hstu_attn_bwd(dims, seq, qkv[:, :hq], qkv[:, hq:2 * hq], qkv[:, 2 * hq:], g,
                                 row_stride=qkv.stride(0), rab_pos=rp, rab_time=rt, workspace=ws,
                                 stream=stream)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = sum(10 * dh * H * int(n) * (int(n) + 1) // 2 for n in w.seq.lengths)
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": f"attention gradients dQ, dK, dV, 8 x 8192 tokens, {H} heads x {dh}, "
                        "causal, rab pos+time",
            "ms": round(ms, 4), "algorithmic_flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_MFMA_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_MFMA_TFLOPS, 4)},
            "note": "time of one hstu_attn_bwd call (schedule, dQ kernel, dK/dV kernel), "
                    "HIP events on the launch stream"}


def layer_bwd_measure(torch, np, ops, dev, wl, reps=5):
    """One layer's backward (hstu_layer_bwd: dX and the gradients of w1, b1, w2, b2) on the
    8 x 8192-token batch, d = 1024, 8 heads of 128, for dY drawn N(0, 1) on the device.
    Useful FLOPs: the input and weight gradients of f1 and f2 (2 x 2 T d 2H(dqk+dv) and
    2 x 2 T H dv d) and the attention gradient's five products per allowed pair and head;
    the forward pieces the call recomputes (f1 and the attention) are not counted."""
    w = wl.config(2)
    d = w.dims
    dims, seq = dev.dims_of(d), dev.jagged_of(w.seq)
    rng = np.random.default_rng(1001)
    dw = dev.weights_of(wl.draw_weights(rng, d, bias=True))
    x = dev.bf16_tensor(w.x)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4004)
    d_y = torch.randn((w.seq.total, d.d_model), generator=gen, device="cuda")
    ws = torch.empty(ops.hstu_layer_bwd_workspace_bytes(dims, seq), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def run():
        return ops.hstu_layer_bwd(dims, dw, seq, x, d_y, workspace=ws, stream=stream)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    T, dm, H = w.seq.total, d.d_model, d.num_heads
    n1 = 2 * H * (d.dqk + d.dv)
    att = sum(10 * d.dqk * H * int(n) * (int(n) + 1) // 2 for n in w.seq.lengths)
    flops = 2 * 2 * T * dm * n1 + 2 * 2 * T * H * d.dv * dm + att
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": "layer backward (dX, dw1, db1, dw2, db2), 8 x 8192 tokens, d=1024, "
                        "8 heads x 128, causal, rab pos+time",
            "ms": round(ms, 4), "useful_flops": flops, "tflops": round(tf, 2),
            "pct_mfma_peak": round(100 * tf / PEAK_MFMA_TFLOPS, 2),
            "note": "one hstu_layer_bwd call, HIP events on the launch stream; it recomputes Z, "
                    "U|V|Q|K and the attention output from X (not counted as useful work)"}


def mfalcon_measure(torch, np, ops, dev, wl, n_layers=4, bm=1024, reps=3):
    """M-FALCON serving through an n_layers stack on the 16-user workload: the history
    pass (4096 tokens per user, every layer's K/V kept) and the scoring of 1024
    candidates per user in micro-batches of bm per user, each through all layers against
    the cached history.  Useful FLOPs per candidate and layer: f1 2 d 2H(dqk+dv), attention
    2H(dqk+dv)(n_h + 1) (the history keys and itself), f2 2 H dv d."""
    w = wl.config(4)
    d = w.dims
    rng = np.random.default_rng(4000)
    lw = [w.weights] + [wl.draw_weights(rng, d) for _ in range(n_layers - 1)]
    dims, dw = dev.dims_of(d), [dev.weights_of(x) for x in lw]
    hist = dev.jagged_of(w.seq)
    T_h = w.seq.total
    x_h = dev.bf16_tensor(w.x)
    y_h = torch.empty_like(x_h)
    caches = torch.empty((n_layers, T_h, d.uvqk_width), dtype=torch.float16, device="cuda")
    ws_h = torch.empty(ops.hstu_stack_workspace_bytes(dims, hist), dtype=torch.uint8, device="cuda")
    cand = w.cand
    n_c = int(cand.offsets[1] - cand.offsets[0])
    mbs = []
    for start in range(0, n_c, bm):
        m = min(bm, n_c - start)
        sel = np.concatenate([cand.offsets[b] + start + np.arange(m) for b in range(cand.batch)])
        mc = wl.Jagged(offsets=wl.offsets_from_lengths(np.full(cand.batch, m)),
                       timestamps=cand.timestamps[sel])
        mbs.append((dev.jagged_of(mc), dev.bf16_tensor(w.x_cand[sel])))
    m0 = mbs[0][0]
    ws_c = torch.empty(ops.hstu_stack_mfalcon_workspace_bytes(dims, hist, m0), dtype=torch.uint8,
                       device="cuda")
    y_c = torch.empty((m0.total_tokens, d.d_model), dtype=torch.bfloat16, device="cuda")
    u_c = torch.empty((m0.total_tokens, d.uvqk_width), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()

    def history():
        ops.hstu_stack_fwd(dims, dw, hist, x_h, keep_caches=True, y=y_h, uvqk=caches,
                           workspace=ws_h, stream=stream)

    def score(st=None):
        for mc, xc in mbs:
            ops.hstu_stack_fwd_mfalcon(dims, dw, hist, caches, mc, xc, y_cand=y_c, uvqk_cand=u_c,
                                       workspace=ws_c, stream=st or stream)

    def timed_ms(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    hist_ms = timed_ms(history)
    score_ms = timed_ms(score)
    # the same micro-batch loop captured once in a HIP graph and replayed (the launches of
    # every micro-batch and layer in one submission); checked bit for bit against eager
    score()
    torch.cuda.synchronize()
    y_ref = y_c.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        score(torch.cuda.current_stream())
    y_c.zero_()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(y_c, y_ref), "graph replay differs from the eager micro-batch loop"
    graph_ms = timed_ms(graph.replay)
    # micro-batches spread over 4 streams (default priority), each with its own workspace
    # and outputs: a small micro-batch fills only part of the GPU, and micro-batches are
    # independent of one another
    n_st = min(4, len(mbs))
    streams = [torch.cuda.Stream() for _ in range(n_st)]
    bufs = [(torch.empty_like(ws_c), torch.empty_like(y_c), torch.empty_like(u_c)) for _ in range(n_st)]

    def score_streams():
        ev = torch.cuda.Event()
        ev.record(stream)
        for i, (mc, xc) in enumerate(mbs):
            st = streams[i % n_st]
            st.wait_event(ev)
            wsb, yb, ub = bufs[i % n_st]
            ops.hstu_stack_fwd_mfalcon(dims, dw, hist, caches, mc, xc, y_cand=yb, uvqk_cand=ub,
                                       workspace=wsb, stream=st)
        for st in streams:
            stream.wait_stream(st)

    score_streams()
    torch.cuda.synchronize()
    last = (len(mbs) - 1) % n_st
    assert torch.equal(bufs[last][1], y_ref), "multi-stream scoring differs from the eager loop"
    streams_ms = timed_ms(score_streams)
    H, dq, dv_, dm = d.num_heads, d.dqk, d.dv, d.d_model
    n_h = int(w.seq.lengths[0])
    n_cand = int(cand.total)
    per_cand = 2 * dm * 2 * H * (dq + dv_) + 2 * H * (dq + dv_) * (n_h + 1) + 2 * H * dv_ * dm
    f1, att, f2 = useful_flops(w.seq.lengths.tolist(), dm, H, dq, dv_)
    return {"workload": f"M-FALCON serving, {cand.batch} users x ({n_h} history + {n_c} "
                        f"candidates), d={dm}, {H} heads x {dq}, {n_layers}-layer stack, "
                        f"micro-batches of {bm} candidates per user",
            "layers": n_layers, "b_m": bm, "history_ms": round(hist_ms, 3),
            "history_tflops": round(n_layers * (f1 + att + f2) / (hist_ms * 1e-3) / 1e12, 1),
            "score_ms": round(score_ms, 3),
            "candidates_per_s": round(n_cand / (score_ms * 1e-3), 1),
            "score_ms_graph": round(graph_ms, 3),
            "candidates_per_s_graph": round(n_cand / (graph_ms * 1e-3), 1),
            "score_ms_4_streams": round(streams_ms, 3),
            "candidates_per_s_4_streams": round(n_cand / (streams_ms * 1e-3), 1),
            "score_tflops": round(n_layers * n_cand * per_cand / (score_ms * 1e-3) / 1e12, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=24)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run 4 device-to-device copies of this many bytes (counter "
                         "calibration for HBM traffic) and exit")
    ap.add_argument("--traffic-record", metavar="DIR", default=None,
                    help="only write profiles/attention_traffic.json from the rocprofv3 counter "
                         "databases DIR/{pmc_fetch,pmc_write,pmc_cfetch,pmc_cwrite}/pmc_results.db "
                         "(attention FETCH_SIZE / WRITE_SIZE, then the same counters over a "
                         "--copy-bytes run) and exit")
    args = ap.parse_args()
    if args.traffic_record:
        write_traffic_record(args.traffic_record, args.copy_bytes or (1 << 30))
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); the jagged batch would "
              "shard by sequence with no exchange across GPUs, which this build does not run.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from hstu_pointwise_attention_jagged_amd import device as dev
    from hstu_pointwise_attention_jagged_amd import ops
    from hstu_pointwise_attention_jagged_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_bytes:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings give the
        # bytes-per-count scale of those counters
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_bytes} bytes 4 times")
        return
    log("building inputs (8 x 8192 tokens, d=1024, 8x128 heads)")
    w = wl.config(2)
    d = w.dims
    dims = dev.dims_of(d)
    seq = dev.jagged_of(w.seq)
    T = w.seq.total
    rng = np.random.default_rng(1000)
    layer_w = [dev.weights_of(w.weights)]
    for _ in range(args.layers - 1):
        layer_w.append(dev.weights_of(wl.draw_weights(rng, d)))
    x0 = dev.bf16_tensor(w.x)
    bufs = [torch.empty_like(x0)]
    uvqk = torch.empty((T, d.uvqk_width), dtype=torch.float16, device="cuda")
    ws = torch.empty(ops.hstu_stack_workspace_bytes(dims, seq), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        # the whole stack in one call: the batch's schedule is built once, then every
        # layer runs f1, attention, norm-gate and f2
        y, _ = ops.hstu_stack_fwd(dims, layer_w, seq, x0, y=bufs[0], uvqk=uvqk, workspace=ws,
                                  stream=stream)
        return y

    log(f"warmup {args.warmup} steps of {args.layers} layers")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ops.profile_reset()
    ops.profile_enable(True)
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ops.profile_enable(False)
    kern = ops.profile_collect()
    ops.profile_reset()

    lengths = w.seq.lengths.tolist()
    f1, att, f2 = useful_flops(lengths, d.d_model, d.num_heads, d.dqk, d.dv)
    flops_step = (f1 + att + f2) * args.layers
    ms = elapsed / args.steps * 1e3
    tflops = flops_step / (elapsed / args.steps) / 1e12

    att_ms, att_n = kern["attention"]
    att_avg_ms = att_ms / max(att_n, 1)
    achieved = att / (att_avg_ms * 1e-3) / 1e12
    per_kernel = {k: round(v[0] / max(v[1], 1), 4) for k, v in kern.items()}
    traffic = traffic_record()
    log(f"step {ms:.2f} ms, {tflops:.1f} TFLOP/s; per-kernel avg ms {per_kernel}")

    out = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 I/O and f1/f2 operands, fp16 attention operands, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": f"uniform 8x8192 jagged batch, d=1024, 8 heads x 128, causal, "
                               f"rab pos+time, {args.layers}-layer stack",
                   "batch": 8, "seq_len": 8192, "d_model": 1024, "num_heads": 8, "head_dim": 128,
                   "layers": args.layers, "parallelism": "single GPU"},
        "pct_mfma_peak": round(100 * tflops / PEAK_MFMA_TFLOPS, 2),
        "useful_tflop_per_layer": round((f1 + att + f2) / 1e12, 4),
        "kernel_avg_ms": per_kernel,
        "roofline": {"kernel": "attention", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
                     "traffic": traffic,
                     "algorithmic_flops_per_launch": att, "avg_launch_ms": round(att_avg_ms, 4)},
        "cpu_baseline": None,
        "host": platform.node(),
    }
    log("stochastic length on the 128-user raw batch")
    out["stochastic_length"] = sl_measure(torch, np, ops, dev, wl)
    log("M-FALCON serving through a 4-layer stack, micro-batches of 1024 and 128 per user")
    out["mfalcon_serving"] = [mfalcon_measure(torch, np, ops, dev, wl, bm=bm) for bm in (1024, 128)]
    log("attention gradients (dQ, dK, dV) on the 8 x 8192 batch")
    out["attention_backward"] = bwd_measure(torch, np, ops, dev, wl)
    log("layer backward on the 8 x 8192 batch")
    out["layer_backward"] = layer_bwd_measure(torch, np, ops, dev, wl)
    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle, one layer on two 8192-token sequences")
        out["cpu_baseline"] = cpu_baseline(w, args.layers)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
