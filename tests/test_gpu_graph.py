"""HIP graph capture of the library's entry points.

The entry points allocate nothing, synchronise nothing and clear memory with kernels (no
memset), so a caller may capture them in a graph and replay it: a serving loop of
M-FALCON micro-batches, a training step's layer.  Each test captures a call on
pre-allocated buffers, then replays the graph three times with the program's own eager
work and synchronisations in between, and checks every replay bit for bit against the
eager result (the output buffer is cleared before each replay, so the replay must
rewrite it).
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from hstu_pointwise_attention_jagged_amd import device as dev  # noqa: E402
from hstu_pointwise_attention_jagged_amd import ops  # noqa: E402
from hstu_pointwise_attention_jagged_amd import workloads as wl  # noqa: E402

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _replay_and_check(graph, outputs, refs, eager):
    for r in range(3):
        for o in outputs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outputs, refs):
            assert torch.equal(o, ref), f"replay {r} differs from the eager result"
        eager()  # the program's own work between replays
        torch.cuda.synchronize()


def test_layer_forward_in_a_graph():
    w = wl.config(1, batch=16)
    d = w.dims
    dims, seq, dw = dev.dims_of(d), dev.jagged_of(w.seq), dev.weights_of(w.weights)
    x = dev.bf16_tensor(w.x)
    y = torch.empty((w.seq.total, d.d_model), dtype=torch.bfloat16, device="cuda")
    uvqk = torch.empty((w.seq.total, d.uvqk_width), dtype=torch.float16, device="cuda")
    ws = torch.empty(ops.hstu_layer_workspace_bytes(dims, seq), dtype=torch.uint8, device="cuda")
    say(f"[graph] layer forward T={w.seq.total}")
    ops.hstu_layer_fwd(dims, dw, seq, x, y=y, uvqk=uvqk, workspace=ws)
    torch.cuda.synchronize()
    y_ref, u_ref = y.clone(), uvqk.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.hstu_layer_fwd(dims, dw, seq, x, y=y, uvqk=uvqk, workspace=ws,
                           stream=torch.cuda.current_stream())
    _replay_and_check(g, [y, uvqk], [y_ref, u_ref],
                      lambda: ops.hstu_layer_fwd(dims, dw, seq, x))


def test_mfalcon_microbatches_in_a_graph():
    w = wl.config(4, batch=4, seq_len=512)
    d = w.dims
    n_layers = 2
    lw = [dev.weights_of(w.weights),
          dev.weights_of(wl.draw_weights(np.random.default_rng(9), d))]
    dims, hist = dev.dims_of(d), dev.jagged_of(w.seq)
    _, caches = ops.hstu_stack_fwd(dims, lw, hist, dev.bf16_tensor(w.x), keep_caches=True)
    n_c = int(w.cand.offsets[1])
    bm = 64
    mbs = []
    for start in range(0, n_c, bm):
        sel = np.concatenate([w.cand.offsets[b] + start + np.arange(bm) for b in range(w.cand.batch)])
        mc = wl.Jagged(offsets=wl.offsets_from_lengths(np.full(w.cand.batch, bm)),
                       timestamps=w.cand.timestamps[sel])
        mbs.append((dev.jagged_of(mc), dev.bf16_tensor(w.x_cand[sel])))
    T_c = mbs[0][0].total_tokens
    ys = [torch.empty((T_c, d.d_model), dtype=torch.bfloat16, device="cuda") for _ in mbs]
    u_c = torch.empty((T_c, d.uvqk_width), dtype=torch.float16, device="cuda")
    ws = torch.empty(ops.hstu_stack_mfalcon_workspace_bytes(dims, hist, mbs[0][0]),
                     dtype=torch.uint8, device="cuda")
    say(f"[graph] M-FALCON {len(mbs)} micro-batches of {bm} per user, {n_layers} layers")

    def score(stream=None):
        for (mc, xc), y in zip(mbs, ys):
            ops.hstu_stack_fwd_mfalcon(dims, lw, hist, caches, mc, xc, y_cand=y, uvqk_cand=u_c,
                                       workspace=ws, stream=stream)

    score()
    torch.cuda.synchronize()
    refs = [y.clone() for y in ys]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        score(torch.cuda.current_stream())
    _replay_and_check(g, ys, refs, lambda: ops.hstu_stack_fwd(dims, lw, hist, dev.bf16_tensor(w.x)))


def test_attention_backward_in_a_graph():
    rng = np.random.default_rng(21)
    seq = wl.jagged_from_lengths(rng, [300, 0, 77, 129])
    H, dh = 2, 64
    dims = ops.LayerDims(d_model=128, num_heads=H, dqk=dh, dv=dh)
    qkv = dev.f16_tensor(wl.round_f16(0.3 * rng.standard_normal((seq.total, 3 * H * dh),
                                                              dtype=np.float32)))
    g_out = torch.from_numpy(rng.standard_normal((seq.total, H * dh)).astype(np.float32)).cuda()
    P = torch.from_numpy((0.3 * rng.standard_normal((1, 64))).astype(np.float32)).cuda()
    Tt = torch.from_numpy((0.3 * rng.standard_normal((1, 32))).astype(np.float32)).cuda()
    js = dev.jagged_of(seq)
    hq = H * dh
    ws = torch.empty(ops.hstu_attn_bwd_workspace_bytes(dims, js), dtype=torch.uint8, device="cuda")
    say(f"[graph] attention backward T={seq.total}")

    def run(stream=None):
        return ops.hstu_attn_bwd(dims, js, qkv[:, :hq], qkv[:, hq:2 * hq], qkv[:, 2 * hq:], g_out,
                                 row_stride=qkv.stride(0), rab_pos=P, rab_time=Tt, rab_grads=True,
                                 workspace=ws, stream=stream)

    refs = run()
    torch.cuda.synchronize()
    refs = [t.clone() for t in refs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run(torch.cuda.current_stream())
    _replay_and_check(g, list(outs), refs, lambda: run())
