"""Rounding-point budget of the layer (CPU only).

Emulates, in float64, where the GPU path rounds: the f1 output U|V|Q|K, the attention
weights A before the P.V product, the f2 operand G and Y.  In the built path the attention
leaves each head's output standardised with its own mean and variance (fp16), and f2 forms
G = ((o - mu) rstd) U from those parts in fp16 steps (the head factors a_h, b_h rounded,
one rounding per fused multiply-add, one for the product with U) against w2 in fp16.  The
attention kernel carries scores scaled by -log2(e) (Q rounded once more after that
scaling, weights t / (1 + 2^t) rounded, -ln 2 applied to the output), and the emulation
takes the same steps.  Blocks whose bias is one constant get it through an fp16 MFMA
operand; the emulation rounds every scaled bias value to fp16 (an upper bound).  It
checks that the built precision (fp16 U|V|Q|K and A, bf16 G and Y) stays within the
layer's tolerance with margin, and records that rounding U|V|Q|K and A to bf16 instead
costs markedly more error -- the reason those operands are fp16.  Inputs are the seeded
Zipf workload (32 users to keep the run short).
"""

import numpy as np
import pytest

from hstu_pointwise_attention_jagged_amd import workloads as wl
from oracle import hstu_ref as ref

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def _bf16(x):
    return wl.round_bf16(np.asarray(x, np.float32)).astype(np.float64)


def _f16(x):
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def _ident(x):
    return x


L2E, LN2 = 1.4426950408889634, 0.6931471805599453


def _gate_fp16(o, u, H, dh, eps):
    """G as the fused f2 staging forms it (no affine): per-head standardised fp16 parts,
    the row's LayerNorm statistics combined from the heads' exactly, fp16 arithmetic."""
    T = o.shape[0]
    oh = o.reshape(T, H, dh)
    mu_h = oh.mean(axis=2)
    var_h = ((oh - mu_h[..., None]) ** 2).mean(axis=2)
    inv = np.where(var_h > 0, 1.0 / np.sqrt(np.where(var_h > 0, var_h, 1.0)), 0.0)
    c = _f16((oh - mu_h[..., None]) * inv[..., None])
    mu = mu_h.mean(axis=1)
    var = (var_h + (mu_h - mu[:, None]) ** 2).mean(axis=1)
    rstd = 1.0 / np.sqrt(var + eps)
    a = _f16(np.sqrt(var_h) * rstd[:, None])
    b = _f16((mu_h - mu[:, None]) * rstd[:, None])
    t = _f16(c * a[..., None] + b[..., None])
    return _f16(t.reshape(T, H * dh) * u)


def _emulate(w, r_uvqk, r_a, r_g, r_y, fold=False, fused_gate=False):
    d = w.dims
    H, dh = d.num_heads, d.dqk
    u, v, q, k = (r_uvqk(t) for t in ref.f1_split(w.x, w.weights.w1, None, H, dh, dh))
    o = np.zeros((w.seq.total, H * dh))
    off = w.seq.offsets
    ts = w.seq.timestamps.astype(np.int64)
    P = w.weights.rab_pos[0].astype(np.float64)
    Tt = w.weights.rab_time[0].astype(np.float64)
    for b in range(w.seq.batch):
        s0, s1 = off[b], off[b + 1]
        n = s1 - s0
        if n == 0:
            continue
        i = np.arange(n)
        bias = P[ref.pos_bucket(np.maximum(i[:, None] - i[None, :], 0), 64)] + \
            Tt[ref.time_bucket(ts[s0:s1][:, None], ts[s0:s1][None, :], 32)]
        mask = i[None, :] <= i[:, None]
        for h in range(H):
            c = slice(h * dh, (h + 1) * dh)
            if fold:
                qs = r_uvqk(-L2E * q[s0:s1, c])
                t = qs @ k[s0:s1, c].T + r_uvqk(-L2E * bias)
                a = r_a(np.where(mask, t / (1.0 + np.exp2(t)), 0.0))
                o[s0:s1, c] = -LN2 * (a @ v[s0:s1, c])
            else:
                a = r_a(np.where(mask, ref.silu(q[s0:s1, c] @ k[s0:s1, c].T + bias), 0.0))
                o[s0:s1, c] = a @ v[s0:s1, c]
    if fused_gate:
        g = _gate_fp16(o, u, H, dh, d.ln_eps)
        return r_y(g @ _f16(w.weights.w2).T)
    g = r_g(ref.norm_gate(o, u, None, None, d.ln_eps))
    return r_y(g @ w.weights.w2.T.astype(np.float64))


@pytest.fixture(scope="module")
def case():
    w = wl.config(1, batch=32)
    exact = _emulate(w, _ident, _ident, _ident, _ident)
    want = ref.layer_fwd(w.x, w.weights, w.seq.offsets, w.seq.timestamps, 4, 64, 64)
    np.testing.assert_allclose(exact, want, rtol=1e-9, atol=1e-9)  # emulator == oracle
    folded = _emulate(w, _ident, _ident, _ident, _ident, fold=True)
    np.testing.assert_allclose(folded, want, rtol=1e-9, atol=1e-9)  # the scaling is exact
    return w, exact


def test_built_precision_meets_tolerance_with_margin(case):
    w, exact = case
    err = np.abs(_emulate(w, _f16, _f16, None, _bf16, fold=True, fused_gate=True) - exact)
    assert err.max() <= 0.8 * MAX_ABS
    assert err.mean() <= 0.7 * MEAN_ABS
    # the fused fp16 gate costs no more than rounding a separately formed G to bf16
    sep = np.abs(_emulate(w, _f16, _f16, _bf16, _bf16, fold=True) - exact)
    assert err.mean() <= sep.mean() * 1.02


def test_bf16_attention_operands_cost_more(case):
    w, exact = case
    built = np.abs(_emulate(w, _f16, _f16, None, _bf16, fold=True, fused_gate=True) - exact)
    all_bf16 = np.abs(_emulate(w, _bf16, _bf16, _bf16, _bf16) - exact)
    assert all_bf16.mean() > 1.4 * built.mean()
    assert all_bf16.max() > built.max()
