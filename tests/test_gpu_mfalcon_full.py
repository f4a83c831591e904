"""M-FALCON at the full serving shape: 16 users, each a 4096-token history plus 1024
candidates, d = 512, 8 heads of 64 (ltzyclt.github.io section 5.2: candidates scored in
micro-batches of b_m against the cached history; chenhuiyu.github.io, section
"另外三块拼图", item 3: 1024 candidates per user).

Bars: micro-batches of 1024 and of 128 candidates per user give bitwise-equal outputs;
sampled history rows and sampled candidates of every user match the fp64 oracle within
max-abs 2e-2 and mean-abs 2e-3; a 4-layer stack equals sequential per-layer calls bit
for bit.  The history is longer than one block table of the attention kernel (2048
keys), so prefix blocks past that point are exercised.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from hstu_pointwise_attention_jagged_amd import device as dev  # noqa: E402
from hstu_pointwise_attention_jagged_amd import ops  # noqa: E402
from hstu_pointwise_attention_jagged_amd import workloads as wl  # noqa: E402
from oracle import hstu_ref as ref  # noqa: E402

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def work():
    w = wl.config(4)
    assert w.seq.batch == 16 and int(w.seq.lengths[0]) == 4096 and int(w.cand.lengths[0]) == 1024
    return w


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


def _microbatches(cand, bm):
    n_c = int(cand.offsets[1] - cand.offsets[0])
    for start in range(0, n_c, bm):
        m = min(bm, n_c - start)
        sel = np.concatenate([cand.offsets[b] + start + np.arange(m) for b in range(cand.batch)])
        mc = wl.Jagged(offsets=wl.offsets_from_lengths(np.full(cand.batch, m)),
                       timestamps=cand.timestamps[sel])
        yield sel, mc


def _score(dims, wts, hist, uvqk_h, w, bm):
    out = np.zeros((w.cand.total, w.dims.d_model), np.int16)
    for sel, mc in _microbatches(w.cand, bm):
        y_c, _ = ops.hstu_layer_fwd_mfalcon(dims, wts, hist, uvqk_h, dev.jagged_of(mc),
                                            dev.bf16_tensor(w.x_cand[sel]))
        torch.cuda.synchronize()
        out[sel] = _bits(y_c)
    return out


def test_mfalcon_full_shape_microbatch_bitwise_and_oracle(work):
    w = work
    d = w.dims
    dims, wts, hist = dev.dims_of(d), dev.weights_of(w.weights), dev.jagged_of(w.seq)
    say(f"[mfalcon full] B={w.seq.batch} hist={w.seq.lengths[0]} cand={w.cand.lengths[0]} "
        f"d={d.d_model} H={d.num_heads}x{d.dqk}")
    y_h, uvqk_h = ops.hstu_layer_fwd(dims, wts, hist, dev.bf16_tensor(w.x))
    torch.cuda.synchronize()
    y1024 = _score(dims, wts, hist, uvqk_h, w, 1024)
    y128 = _score(dims, wts, hist, uvqk_h, w, 128)
    assert np.array_equal(y1024, y128), "b_m = 1024 and b_m = 128 differ"
    say("        b_m 1024 == b_m 128 bitwise")

    # oracle: history K, V once, then sampled rows (every user)
    rng = np.random.default_rng(44)
    H, dh = d.num_heads, d.dqk
    u, v, q, k = ref.f1_split(w.x, w.weights.w1, w.weights.b1, H, dh, dh)
    off = w.seq.offsets
    h_rows = sorted({int(off[b] + r) for b in range(w.seq.batch)
                     for r in (0, 127, 2047, 2048, 2100 + b, 4095, int(rng.integers(0, 4096)))})
    o_h = ref.attention(q, k, v, off, w.seq.timestamps, H, dh, dh, w.weights.rab_pos,
                        w.weights.rab_time, rows=h_rows)
    want_h = ref.f2(ref.norm_gate(o_h[h_rows], u[h_rows], w.weights.ln_gamma, w.weights.ln_beta,
                                  d.ln_eps), w.weights.w2, w.weights.b2)
    got_h = dev.bf16_to_numpy(y_h).astype(np.float64)[h_rows]
    err = np.abs(got_h - want_h)
    say(f"        history rows ({len(h_rows)}): max_abs={err.max():.3e} mean_abs={err.mean():.3e}")
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS

    coff = w.cand.offsets
    c_rows = sorted({int(coff[b] + r) for b in range(w.cand.batch)
                     for r in (0, 1, 127, 128, 1023, int(rng.integers(0, 1024)))})
    uc, vc, qc, kc = ref.f1_split(w.x_cand[c_rows], w.weights.w1, w.weights.b1, H, dh, dh)
    # the sampled candidates as a jagged batch of their own (a candidate's result does not
    # depend on the other candidates of its micro-batch)
    users = np.searchsorted(coff, np.array(c_rows), side="right") - 1
    sub = wl.Jagged(offsets=wl.offsets_from_lengths(np.bincount(users, minlength=w.cand.batch)),
                    timestamps=w.cand.timestamps[c_rows])
    o_c = ref.attention(qc, kc, vc, sub.offsets, sub.timestamps, H, dh, dh, w.weights.rab_pos,
                        w.weights.rab_time, prefix=(k, v, off, w.seq.timestamps),
                        mask=ref.SELF_ONLY)
    want_c = ref.f2(ref.norm_gate(o_c, uc, w.weights.ln_gamma, w.weights.ln_beta, d.ln_eps),
                    w.weights.w2, w.weights.b2)
    got_c = wl.bf16_to_f32(y1024[c_rows].view(np.uint16)).astype(np.float64)
    err = np.abs(got_c - want_c)
    say(f"        candidates ({len(c_rows)}): max_abs={err.max():.3e} mean_abs={err.mean():.3e}")
    assert np.all(np.isfinite(got_c))
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS


def test_mfalcon_full_shape_stack_equals_sequential_layers(work):
    w = work
    d = w.dims
    n_layers = 4
    rng = np.random.default_rng(303)
    lw = [w.weights] + [wl.draw_weights(rng, d) for _ in range(n_layers - 1)]
    dims, hist = dev.dims_of(d), dev.jagged_of(w.seq)
    dw = [dev.weights_of(x) for x in lw]
    say(f"[mfalcon full stack] {n_layers} layers")
    _, caches = ops.hstu_stack_fwd(dims, dw, hist, dev.bf16_tensor(w.x), keep_caches=True)
    outs = {}
    for bm in (1024, 128):
        o = np.zeros((w.cand.total, d.d_model), np.int16)
        for sel, mc in _microbatches(w.cand, bm):
            yc = ops.hstu_stack_fwd_mfalcon(dims, dw, hist, caches, dev.jagged_of(mc),
                                            dev.bf16_tensor(w.x_cand[sel]))
            torch.cuda.synchronize()
            o[sel] = _bits(yc)
        outs[bm] = o
    assert np.array_equal(outs[1024], outs[128]), "b_m changed the stack's result"
    # per-layer calls on micro-batches of 1024
    seq_out = np.zeros_like(outs[1024])
    for sel, mc in _microbatches(w.cand, 1024):
        cs = dev.jagged_of(mc)
        xc = dev.bf16_tensor(w.x_cand[sel])
        for l in range(n_layers):
            xc, _ = ops.hstu_layer_fwd_mfalcon(dims, dw[l], hist, caches[l], cs, xc)
        torch.cuda.synchronize()
        seq_out[sel] = _bits(xc)
    assert np.array_equal(seq_out, outs[1024]), "stack differs from sequential M-FALCON layers"
    assert np.all(np.isfinite(wl.bf16_to_f32(outs[1024].view(np.uint16))))
