"""Benchmark: jagged HSTU layer forward on one MI355X.

A step is one forward pass of a 24-layer HSTU stack (independent random weights per
layer, Y of layer l is X of layer l+1) over the 8 x 8192-token batch, d = 1024, 8 heads
of 128, causal mask with positional + log-time relative bias: every kernel of the hot
path (jagged schedule, f1 + SiLU, pointwise attention, f2 with LayerNorm + gate) runs once
per layer.  Inputs and weights are resident in HBM before the timed region.

Prints one JSON line on stdout; progress goes to stderr.

Besides the step, the line carries separate measurements of Stochastic Length, M-FALCON
serving, the attention gradients (hstu_attn_bwd) and one layer's backward (hstu_layer_bwd).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers 24] [--no-cpu-baseline]
                  [--only-step] [--only-backward]
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
PEAK_FLOP_PER_CLOCK = 256 * 4 * 1024  # CUs x SIMDs x dense fp16/bf16 MFMA FLOP per clock
COUNTER_RECORD = os.path.join(ROOT, "profiles", "layer_counters.json")
CSRC = os.path.join(ROOT, "hstu_pointwise_attention_jagged_amd", "csrc")


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


# the sources the forward layer's kernels (f1 with the f2 operand preparation, attention, f2) are
# compiled from, with the headers they include and the host code that launches them
_LAYER_KERNEL_SOURCES = ("attention.hip", "gemm.hip", "common.h", "kernels.h", "api.cpp")


def _kernel_sources_sha():
    """sha256 of the kernel sources a counter record describes."""
    h = hashlib.sha256()
    for name in _LAYER_KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def counter_record():
    """The committed counter record, if the kernel sources are unchanged since it was taken."""
    try:
        with open(COUNTER_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sources_sha256") != _kernel_sources_sha():
        return None  # kernels changed since the counters were taken
    return rec


# kernels of one c2 layer: (label, name substring, useful FLOPs, algorithmic HBM bytes)
def _layer_kernels():
    T, d, H, dh = 65536, 1024, 8, 128
    n1 = 2 * H * 2 * dh
    f1, att, f2 = useful_flops([8192] * 8, d, H, dh, dh)
    return [
        # f1 with the f2 operand conversion in its tail (w2 read as bf16, written as fp16)
        ("f1 GEMM + SiLU", "gemm256_kernel<0, 0, 1, 1>", f1, 2 * (T * d + n1 * d + T * n1) + 2 * 2 * d * H * dh),
        ("attention", "attn_kernel<128, 0, 4", att, 2 * 3 * T * H * dh + 2 * T * H * dh + 8 * T * H),
        ("f2 GEMM with LayerNorm + gate", "gate_gemm_tab_kernel", f2,
         2 * 2 * T * H * dh + 8 * T * H + 2 * d * H * dh + 2 * T * d),
    ]


def _read_pmc(path):
    """{kernel name: {counter: [values per dispatch]}, ...} and durations (ns) per name."""
    import csv
    vals, durs = {}, {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            vals.setdefault(name, {}).setdefault(r["Counter_Name"], {})[r["Dispatch_Id"]] = float(r["Counter_Value"])
            durs.setdefault(name, {})[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    avg = lambda d: sum(d.values()) / max(len(d), 1)
    return ({n: {c: avg(v) for c, v in cs.items()} for n, cs in vals.items()},
            {n: avg(d) for n, d in durs.items()})


def write_counter_record(d, copy_bytes, out_path=None):
    """Per-kernel counter summary of one c2 layer from the rocprofv3 --pmc passes under d:
    sq1, sq2 (SQ and GRBM counters), fetch, write (FETCH_SIZE, WRITE_SIZE) over
    `bench.py --layers 1 --steps 1 --warmup 1 --only-step`, and cfetch, cwrite (the same
    two counters over `bench.py --copy-bytes copy_bytes`), all in CSV."""
    runs = {k: _read_pmc(os.path.join(d, k, "pmc_counter_collection.csv"))
            for k in ("sq1", "sq2", "fetch", "write", "cfetch", "cwrite")}
    copy = lambda k, c: [v[c] for n, v in runs[k][0].items() if "copyBuffer" in n][0]
    fetch_scale = copy_bytes / (1024.0 * copy("cfetch", "FETCH_SIZE"))
    write_scale = copy_bytes / (1024.0 * copy("cwrite", "WRITE_SIZE"))
    simds = 256 * 4
    kernels = {}
    for label, sub, flops, alg in _layer_kernels():
        def pick(k, c):
            for n, v in runs[k][0].items():
                if sub in n and c in v:
                    return v[c], runs[k][1][n]
            return None, None
        gui, dur = pick("sq1", "GRBM_GUI_ACTIVE")
        if gui is None:
            continue
        xcds = 8  # GRBM_GUI_ACTIVE adds up the 8 XCDs' busy cycles
        clk = gui / xcds / dur  # GHz
        cyc = dur * clk  # shader cycles over the dispatch
        g = lambda k, c: pick(k, c)[0] or 0.0
        mfma = g("sq1", "SQ_INSTS_MFMA")
        rec = {"ms": dur / 1e6, "clock_ghz": clk,
               "mfma_busy_frac": g("sq1", "SQ_VALU_MFMA_BUSY_CYCLES") / (simds * cyc),
               "valu_busy_frac": 4 * g("sq1", "SQ_ACTIVE_INST_VALU") / (simds * cyc),
               "sq_busy_frac": g("sq1", "SQ_BUSY_CYCLES") / (32 * cyc),
               "mfma_insts": mfma,
               "valu_per_mfma": (g("sq2", "SQ_INSTS_VALU") - mfma) / mfma if mfma else None,
               "trans_per_mfma": g("sq2", "SQ_INSTS_VALU_TRANS_F32") / mfma if mfma else None,
               "salu_per_mfma": g("sq2", "SQ_INSTS_SALU") / mfma if mfma else None,
               "lds_per_mfma": g("sq2", "SQ_INSTS_LDS") / mfma if mfma else None,
               "lds_bank_conflict_frac": (g("sq2", "SQ_LDS_BANK_CONFLICT") / g("sq2", "SQ_ACTIVE_INST_LDS")
                                          if g("sq2", "SQ_ACTIVE_INST_LDS") else None),
               "fetch_bytes": 1024.0 * g("fetch", "FETCH_SIZE") * fetch_scale,
               "write_bytes": 1024.0 * g("write", "WRITE_SIZE") * write_scale,
               "algorithmic_bytes": alg, "useful_flops": flops}
        rec["hbm_gbs"] = (rec["fetch_bytes"] + rec["write_bytes"]) / dur
        rec["tflops"] = flops / dur / 1e3 if flops else None
        rec["peak_tflops_at_clock"] = PEAK_FLOP_PER_CLOCK * clk / 1e3
        kernels[label] = rec
    out = {"workload": "one layer, 8 x 8192 tokens, d=1024, 8 heads x 128, causal, rab pos+time",
           "kernel_sources_sha256": _kernel_sources_sha(), "copy_bytes": copy_bytes,
           "fetch_scale": fetch_scale, "write_scale": write_scale, "kernels": kernels}
    out_path = out_path or COUNTER_RECORD
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    log(f"wrote {out_path}")
    hdr = ("| kernel | ms | clock GHz | TFLOP/s | % of peak at that clock | MFMA busy | VALU busy | "
           "VALU / MFMA | trans / MFMA | SALU / MFMA | LDS / MFMA | HBM fetch + write MB | "
           "algorithmic MB | HBM GB/s |")
    print(hdr)
    print("|" + "---|" * 14)
    for k, r in kernels.items():
        f = lambda x, p=2: "-" if x is None else f"{x:.{p}f}"
        pct = None if not r["tflops"] else 100 * r["tflops"] / r["peak_tflops_at_clock"]
        print(f"| {k} | {r['ms']:.4f} | {r['clock_ghz']:.2f} | {f(r['tflops'], 0)} | {f(pct, 1)} | "
              f"{100 * r['mfma_busy_frac']:.1f}% | {100 * r['valu_busy_frac']:.1f}% | {f(r['valu_per_mfma'])} | "
              f"{f(r['trans_per_mfma'])} | {f(r['salu_per_mfma'])} | {f(r['lds_per_mfma'])} | "
              f"{(r['fetch_bytes'] + r['write_bytes']) / 1e6:.0f} | {r['algorithmic_bytes'] / 1e6:.0f} | "
              f"{r['hbm_gbs']:.0f} |")


def host_info():
    """CPU model, visible logical CPUs and numpy's BLAS library with its thread count."""
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    info = {"cpu_model": model, "logical_cpus_visible": os.cpu_count(),
            "cpus_in_affinity": len(os.sched_getaffinity(0))}
    try:
        import numpy  # noqa: F401  (loads the BLAS library that threadpoolctl reports)
        import threadpoolctl
        info["blas"] = [{k: p.get(k) for k in ("internal_api", "version", "num_threads",
                                               "threading_layer", "architecture")}
                        for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
    except Exception as e:  # threadpoolctl missing or failing: say so
        info["blas"] = f"unavailable ({type(e).__name__})"
    return info


# Host threads the oracle may use: one GPU's share of the host cores (16), or fewer when
# fewer are available to the process.
CPU_SHARE_PER_GPU = 16


def cpu_baseline(w, layers, n_seq=2):
    """fp64 oracle on the first n_seq 8192-token sequences of the same batch, one layer.
    Its attention runs on a pool of `cores` threads; its matrix products run in numpy's
    BLAS, whose own thread count is reported with the host description."""
    import numpy as np
    from oracle import hstu_ref

    d = w.dims
    cores = min(len(os.sched_getaffinity(0)), CPU_SHARE_PER_GPU)
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
            "kind": "oracle", "host": host_info(),
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


def _events_ms(torch, stream, fn, reps):
    """Average time of fn over reps calls, HIP events on the launch stream."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _kernel_ms(torch, ops, fn, reps=3):
    """Per-kernel average times (ms) of fn from the library's event timing (run untimed)."""
    torch.cuda.synchronize()
    ops.profile_reset()
    ops.profile_enable(True)
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    ops.profile_enable(False)
    k = ops.profile_collect()
    ops.profile_reset()
    return {n: round(v[0] / v[1], 4) for n, v in k.items() if v[1]}


def attention_by_layer(torch, ops, dims, layer_w, seq, x0, stream, every=4):
    """The stack's layers run one call at a time (outside the timed region): for every
    `every`-th layer, the attention launch's time, the shader clock during it and the
    standard deviation of the layer's input.  With no residual path the activations shrink
    layer by layer, and the attention's clock rises as its operands draw less power."""
    rows = []
    x = x0
    for l, wt in enumerate(layer_w):
        keep = l % every == 0 or l == len(layer_w) - 1
        if keep:
            torch.cuda.synchronize()
            ops.profile_reset()
            ops.profile_enable(True, kernels=["attention"])
        y, _ = ops.hstu_layer_fwd(dims, wt, seq, x, stream=stream)
        if keep:
            torch.cuda.synchronize()
            ops.profile_enable(False)
            ms, n = ops.profile_collect()["attention"]
            rows.append({"layer": l, "attention_ms": round(ms / max(n, 1), 4),
                         "clock_ghz": round(ops.profile_clock_ghz(), 3),
                         "input_std": float(f"{float(x.float().std()):.3g}")})
            ops.profile_reset()
        x = y
    torch.cuda.synchronize()
    return rows


def zipf_measure(torch, np, ops, dev, wl, layers=24, reps=20):
    """The 64-user batch (lengths truncated Zipf s = 1.2 on [16, 1024], d = 256, 4 heads of
    64): one layer alone and a stack of `layers` layers in one call, useful FLOPs as for
    the main step."""
    w = wl.config(1)
    d = w.dims
    dims, seq = dev.dims_of(d), dev.jagged_of(w.seq)
    rng = np.random.default_rng(1100)
    lw = [dev.weights_of(w.weights)] + [dev.weights_of(wl.draw_weights(rng, d))
                                         for _ in range(layers - 1)]
    x = dev.bf16_tensor(w.x)
    T = w.seq.total
    y = torch.empty_like(x)
    u = torch.empty((T, d.uvqk_width), dtype=torch.float16, device="cuda")
    ws = torch.empty(ops.hstu_stack_workspace_bytes(dims, seq), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def one():
        ops.hstu_layer_fwd(dims, lw[0], seq, x, y=y, uvqk=u, workspace=ws, stream=stream)

    def stack():
        ops.hstu_stack_fwd(dims, lw, seq, x, y=y, uvqk=u, workspace=ws, stream=stream)

    one()
    stack()
    stack()
    torch.cuda.synchronize()
    # medians over three timed groups: a call this short is easily disturbed by one slow
    # launch (a 9 ms stack among 1.7 ms ones has been seen once)
    layer_ms = float(np.median([_events_ms(torch, stream, one, reps) for _ in range(3)]))
    stack_ms = float(np.median([_events_ms(torch, stream, stack, max(reps // 4, 3)) for _ in range(3)]))
    f1, att, f2 = useful_flops(w.seq.lengths.tolist(), d.d_model, d.num_heads, d.dqk, d.dv)
    fl = f1 + att + f2
    return {"workload": f"{w.seq.batch} users, lengths truncated Zipf s=1.2 on [16, 1024] "
                        f"({T} tokens, longest {int(w.seq.lengths.max())}), d={d.d_model}, "
                        f"{d.num_heads} heads x {d.dqk}, causal, rab pos+time",
            "useful_tflop_per_layer": round(fl / 1e12, 6),
            "layer_ms": round(layer_ms, 4), "layer_tflops": round(fl / (layer_ms * 1e-3) / 1e12, 2),
            "stack_layers": layers, "stack_ms": round(stack_ms, 4),
            "stack_tflops": round(layers * fl / (stack_ms * 1e-3) / 1e12, 2),
            "pct_mfma_peak_stack": round(100 * layers * fl / (stack_ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 2),
            "layer_kernel_avg_ms": _kernel_ms(torch, ops, one)}


def sl_layer_measure(torch, np, ops, dev, wl, reps=10):
    """Stochastic Length then one layer on the batch it builds (128 users, raw lengths
    log-uniform on [256, 4096], N = 4096, alpha = 1.6, d = 512, 8 heads of 64), with no
    host copy in between: the layer takes the raw token count as its capacity and reads
    the kept count from the device offsets.  Useful FLOPs count the kept tokens only."""
    w = wl.config(3)
    r = w.raw
    d = w.dims
    dims = dev.dims_of(d)
    raw = dev.jagged_of(r.seq)
    u_keep = torch.from_numpy(r.u_keep.astype(np.float64)).cuda()
    keys = torch.from_numpy(r.keys.view(np.int32)).cuda()
    x = dev.bf16_tensor(r.x)
    wts = dev.weights_of(w.weights)
    T_raw = r.seq.total
    L = int(np.floor(float(r.n_target) ** (r.alpha / 2)))
    max_len = max(L, int(r.seq.lengths.max()))
    stream = torch.cuda.current_stream()
    sl_ws = torch.empty(max(int(ops.hstu_sl_workspace_bytes(raw)), 1), dtype=torch.uint8,
                        device="cuda")
    y = torch.empty((T_raw, d.d_model), dtype=torch.bfloat16, device="cuda")
    u = torch.empty((T_raw, d.uvqk_width), dtype=torch.float16, device="cuda")
    state = {}

    def sl():
        state["sl"] = ops.hstu_stochastic_length(raw, u_keep, keys, x=x, workspace=sl_ws,
                                                 stream=stream)

    sl()
    _, new_off, new_ts, x_out = state["sl"]
    seq = ops.DeviceJagged(offsets=new_off, total_tokens=T_raw, max_seq_len=max_len,
                           timestamps=new_ts)
    lws = torch.empty(ops.hstu_layer_workspace_bytes(dims, seq), dtype=torch.uint8, device="cuda")

    def layer():
        ops.hstu_layer_fwd(dims, wts, seq, x_out, y=y, uvqk=u, workspace=lws, stream=stream)

    def both():
        # SL writes into fresh outputs each call; the layer reads the ones made once above
        # (identical contents: the draws are the same), so the pair runs back to back
        sl()
        layer()

    layer()
    torch.cuda.synchronize()
    both_ms = _events_ms(torch, stream, both, reps)
    layer_ms = _events_ms(torch, stream, layer, reps)
    lengths = np.diff(new_off.cpu().numpy()).tolist()  # after the timed regions
    f1, att, f2 = useful_flops(lengths, d.d_model, d.num_heads, d.dqk, d.dv)
    fl = f1 + att + f2
    return {"workload": f"stochastic length on {r.seq.batch} users (raw lengths log-uniform on "
                        f"[256, 4096], N=4096, alpha=1.6), then one layer on the kept batch, "
                        f"d={d.d_model}, {d.num_heads} heads x {d.dqk}, causal, rab pos+time",
            "raw_tokens": T_raw, "kept_tokens": int(sum(lengths)),
            "useful_tflop_per_layer": round(fl / 1e12, 5),
            "sl_plus_layer_ms": round(both_ms, 4), "layer_ms": round(layer_ms, 4),
            "layer_tflops": round(fl / (layer_ms * 1e-3) / 1e12, 2),
            "pct_mfma_peak_layer": round(100 * fl / (layer_ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 2),
            "layer_kernel_avg_ms": _kernel_ms(torch, ops, layer),
            "note": "one stream, no host synchronisation between SL and the layer; the layer's "
                    "total_tokens is the raw count (a capacity), its kernels read the kept count "
                    "from the device offsets"}


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
    # the training pair: the forward keeps U|V|Q|K and the attention output's parts, and
    # the backward reuses them (only Z is formed again)
    _, uvqk, cn, stats = ops.hstu_layer_fwd_train(dims, dw, seq, x)

    def run_saved():
        return ops.hstu_layer_bwd(dims, dw, seq, x, d_y, workspace=ws, stream=stream,
                                  saved=(uvqk, cn, stats))

    for _ in range(2):
        run_saved()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        run_saved()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_saved = e0.elapsed_time(e1) / reps
    T, dm, H = w.seq.total, d.d_model, d.num_heads
    n1 = 2 * H * (d.dqk + d.dv)
    att = sum(10 * d.dqk * H * int(n) * (int(n) + 1) // 2 for n in w.seq.lengths)
    flops = 2 * 2 * T * dm * n1 + 2 * 2 * T * H * d.dv * dm + att
    tf = flops / (ms * 1e-3) / 1e12
    tf_saved = flops / (ms_saved * 1e-3) / 1e12
    return {"workload": "layer backward (dX, dw1, db1, dw2, db2), 8 x 8192 tokens, d=1024, "
                        "8 heads x 128, causal, rab pos+time",
            "ms": round(ms, 4), "useful_flops": flops, "tflops": round(tf, 2),
            "pct_mfma_peak": round(100 * tf / PEAK_MFMA_TFLOPS, 2),
            "note": "one hstu_layer_bwd call, HIP events on the launch stream; it recomputes Z, "
                    "U|V|Q|K and the attention output from X (not counted as useful work)",
            "saved_activations": {
                "ms": round(ms_saved, 4), "tflops": round(tf_saved, 2),
                "pct_mfma_peak": round(100 * tf_saved / PEAK_MFMA_TFLOPS, 2),
                "note": "one hstu_layer_bwd_saved call on the U|V|Q|K and attention-output parts "
                        "that hstu_layer_fwd_train kept; it recomputes only Z"}}


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
    ap.add_argument("--only-step", action="store_true",
                    help="time the stack only (no side measurements, no CPU baseline): the "
                         "short run that counter collection wraps")
    ap.add_argument("--only-backward", action="store_true",
                    help="only time one layer backward on the 8 x 8192 batch (after two untimed "
                         "calls) and print it: the short run that backward counter collection wraps")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run 4 device-to-device copies of this many bytes (counter "
                         "calibration for HBM traffic) and exit")
    ap.add_argument("--counter-record", metavar="DIR", default=None,
                    help="only write profiles/layer_counters.json (and print its table) from the "
                         "rocprofv3 --pmc CSV passes DIR/{sq1,sq2,fetch,write,cfetch,cwrite} and exit")
    args = ap.parse_args()
    if args.counter_record:
        write_counter_record(args.counter_record, args.copy_bytes or (1 << 30))
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); the library has no "
              "multi-GPU path (the jagged batch would shard by sequence, with no exchange across "
              "GPUs).", file=sys.stderr)
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
    if args.only_backward:
        log("layer backward on the 8 x 8192 batch")
        print(json.dumps({"layer_backward": layer_bwd_measure(torch, np, ops, dev, wl, reps=1)}), flush=True)
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
        # layer runs f1, attention and f2 (LayerNorm and the gate formed in its staging)
        y, _ = ops.hstu_stack_fwd(dims, layer_w, seq, x0, y=bufs[0], uvqk=uvqk, workspace=ws,
                                  stream=stream)
        return y

    log(f"warmup {args.warmup} steps of {args.layers} layers")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Inside the timed steps only the attention launches (the roofline kernel) are
    # bracketed by events; every event pair adds time between launches.
    ops.profile_reset()
    ops.profile_enable(True, kernels=["attention"])
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ops.profile_enable(False)
    kern = ops.profile_collect()
    clock_ghz = ops.profile_clock_ghz()  # average shader clock over the timed attention launches
    ops.profile_reset()
    # the other kernels' averages from one more step, outside the timed region
    per_kernel = _kernel_ms(torch, ops, step, reps=1)
    by_layer = attention_by_layer(torch, ops, dims, layer_w, seq, x0, stream)

    lengths = w.seq.lengths.tolist()
    f1, att, f2 = useful_flops(lengths, d.d_model, d.num_heads, d.dqk, d.dv)
    flops_step = (f1 + att + f2) * args.layers
    ms = elapsed / args.steps * 1e3
    tflops = flops_step / (elapsed / args.steps) / 1e12

    att_ms, att_n = kern["attention"]
    att_avg_ms = att_ms / max(att_n, 1)
    achieved = att / (att_avg_ms * 1e-3) / 1e12
    per_kernel["attention"] = round(att_avg_ms, 4)  # the timed steps' own figure
    rec = counter_record()
    att_rec = (rec or {}).get("kernels", {}).get("attention")
    traffic = att_rec["fetch_bytes"] + att_rec["write_bytes"] if att_rec else None
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
        "dtype": "bf16 I/O and f1 operands, fp16 attention and f2 operands, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": f"uniform 8x8192 jagged batch, d=1024, 8 heads x 128, causal, "
                               f"rab pos+time, {args.layers}-layer stack",
                   "batch": 8, "seq_len": 8192, "d_model": 1024, "num_heads": 8, "head_dim": 128,
                   "layers": args.layers, "parallelism": "single GPU"},
        "pct_mfma_peak": round(100 * tflops / PEAK_MFMA_TFLOPS, 2),
        "useful_tflop_per_layer": round((f1 + att + f2) / 1e12, 4),
        "kernel_avg_ms": per_kernel,  # attention: timed steps; others: one untimed step
        "roofline": {"kernel": "attention", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
                     "traffic": traffic,
                     "algorithmic_flops_per_launch": att, "avg_launch_ms": round(att_avg_ms, 4),
                     # the same peak at the shader clock measured during the timed
                     # attention launches (core-clock against real-time counter in the
                     # kernel; 256 CUs x 4 SIMDs x 1024 FLOP per clock), and the fraction of it
                     "clock_ghz_measured": round(clock_ghz, 3) if clock_ghz else None,
                     "peak_at_measured_clock": round(PEAK_FLOP_PER_CLOCK * clock_ghz / 1e3, 1) if clock_ghz else None,
                     "frac_at_measured_clock": (round(achieved / (PEAK_FLOP_PER_CLOCK * clock_ghz / 1e3), 4)
                                                if clock_ghz else None)},
        "attention_by_layer": by_layer,
        "cpu_baseline": None,
        "host": platform.node(),
    }
    if args.only_step:
        print(json.dumps(out), flush=True)
        return
    log("stochastic length on the 128-user raw batch")
    out["stochastic_length"] = sl_measure(torch, np, ops, dev, wl)
    log("M-FALCON serving through a 4-layer stack, micro-batches of 1024 and 128 per user")
    out["mfalcon_serving"] = [mfalcon_measure(torch, np, ops, dev, wl, bm=bm) for bm in (1024, 128)]
    log("64-user Zipf batch: one layer and a 24-layer stack")
    out["zipf_64_users"] = zipf_measure(torch, np, ops, dev, wl)
    log("stochastic length then a layer on the kept batch, no host copy between")
    out["sl_then_layer"] = sl_layer_measure(torch, np, ops, dev, wl)
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
