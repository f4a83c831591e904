"""Pins of the gradient oracles (CPU only).

oracle/hstu_bwd.attention_bwd must be the derivative of oracle/hstu_ref.attention: every
gradient entry (q, k, v and both bias tables) is compared with a central finite
difference of L = sum(attention(...) * G) for a fixed random G, on small jagged batches
(zero-length, one-token and longer users, shared and per-head tables).  A dropped term,
a wrong sign, a transposed operand or a wrong mask in the gradient fails these checks.
"""

import numpy as np
import pytest

import dataclasses

from hstu_pointwise_attention_jagged_amd import workloads as wl
from oracle import hstu_bwd as bwd
from oracle import hstu_ref as ref


def _case(seed, lengths, H=2, dh=4, per_head_time=True):
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(off[-1])
    ts = np.concatenate([np.cumsum(rng.integers(1, 40, size=n)) if n else np.zeros(0, np.int64)
                         for n in lengths]).astype(np.int64)
    q = rng.standard_normal((T, H * dh))
    k = rng.standard_normal((T, H * dh))
    v = rng.standard_normal((T, H * dh))
    P = 0.5 * rng.standard_normal((1, 6))                       # 6 position buckets
    Tt = 0.5 * rng.standard_normal((H if per_head_time else 1, 5))  # 5 time buckets
    G = rng.standard_normal((T, H * dh))
    return off, ts, q, k, v, P, Tt, G, H, dh


def _loss(off, ts, q, k, v, P, Tt, G, H, dh):
    o = ref.attention(q, k, v, off, ts, H, dh, dh, P, Tt, workers=1)
    return float(np.sum(o * G))


@pytest.mark.parametrize("seed,lengths,per_head", [
    (0, [3, 5, 0, 1, 4], True),
    (1, [9], False),
])
def test_attention_gradient_matches_finite_differences(seed, lengths, per_head):
    off, ts, q, k, v, P, Tt, G, H, dh = _case(seed, lengths, per_head_time=per_head)
    dq, dk, dv, dP, dT = bwd.attention_bwd(q, k, v, G, off, ts, H, dh, dh, P, Tt)
    eps = 1e-6
    args = dict(q=q, k=k, v=v, P=P, Tt=Tt)
    grads = dict(q=dq, k=dk, v=dv, P=dP, Tt=dT)
    for name in args:
        x = args[name]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            a_p = dict(args, **{name: xp})
            a_m = dict(args, **{name: xm})
            num[idx] = (_loss(off, ts, a_p["q"], a_p["k"], a_p["v"], a_p["P"], a_p["Tt"], G, H, dh) -
                        _loss(off, ts, a_m["q"], a_m["k"], a_m["v"], a_m["P"], a_m["Tt"], G, H, dh)) / (2 * eps)
        scale = max(1.0, float(np.abs(num).max()))
        np.testing.assert_allclose(grads[name], num, rtol=0, atol=2e-6 * scale, err_msg=name)


def test_silu_grad_closed_form():
    x = np.array([-30.0, -2.0, -0.5, 0.0, 0.5, 2.0, 30.0])
    s = 1.0 / (1.0 + np.exp(-x))
    np.testing.assert_allclose(bwd.silu_grad(x), s + x * s * (1 - s), rtol=1e-15)
    assert bwd.silu_grad(np.array([0.0]))[0] == 0.5


def test_masked_and_future_tokens_get_no_gradient_from_the_past():
    # the last token's query sees every key; the first token's key is seen by every query,
    # but the first query sees only itself: its dq depends on key 0 alone
    off, ts, q, k, v, P, Tt, G, H, dh = _case(3, [6], per_head_time=False)
    G2 = np.zeros_like(G)
    G2[0] = G[0]  # upstream gradient only on row 0
    dq, dk, dv, _, _ = bwd.attention_bwd(q, k, v, G2, off, ts, H, dh, dh, P, Tt)
    assert np.all(dk[1:] == 0) and np.all(dv[1:] == 0)  # row 0 attends to key 0 only
    assert np.all(dq[1:] == 0)
    assert np.any(dq[0] != 0) and np.any(dk[0] != 0)


def test_sampled_rows_equal_the_full_gradient():
    # the row-sampled path (used at sizes where the full pair matrices do not fit) must
    # give the full gradient's values at the chosen rows and zeros elsewhere
    off, ts, q, k, v, P, Tt, G, H, dh = _case(4, [7, 0, 12, 1, 30])
    full = bwd.attention_bwd(q, k, v, G, off, ts, H, dh, dh, P, Tt)
    rows = [0, 5, 6, 7, 18, 19, 20, 21, 49]
    part = bwd.attention_bwd(q, k, v, G, off, ts, H, dh, dh, P, Tt, rows=rows)
    mask = np.zeros(q.shape[0], dtype=bool)
    mask[rows] = True
    for f, p_ in zip(full[:3], part[:3]):
        np.testing.assert_allclose(p_[mask], f[mask], rtol=1e-12, atol=1e-12)
        assert np.all(p_[~mask] == 0)
    assert part[3] is None and part[4] is None


def _layer_case(seed, lengths, d=8, H=2, dh=4, affine=True, bias=True, per_head=True):
    rng = np.random.default_rng(seed)
    seq = wl.jagged_from_lengths(rng, lengths)
    T = seq.total
    n1 = 2 * H * (dh + dh)
    w = wl.LayerWeights(
        w1=rng.standard_normal((n1, d)) / np.sqrt(d), w2=rng.standard_normal((d, H * dh)) / np.sqrt(H * dh),
        b1=0.3 * rng.standard_normal(n1) if bias else None,
        b2=0.3 * rng.standard_normal(d) if bias else None,
        ln_gamma=1 + 0.2 * rng.standard_normal(H * dh) if affine else None,
        ln_beta=0.2 * rng.standard_normal(H * dh) if affine else None,
        rab_pos=0.3 * rng.standard_normal((H if per_head else 1, 6)),
        rab_time=0.3 * rng.standard_normal((H if per_head else 1, 5)))
    x = rng.standard_normal((T, d))
    G = rng.standard_normal((T, d))
    return seq, w, x, G, H, dh


def _layer_loss(seq, w, x, G, H, dh):
    y = ref.layer_fwd(x, w, seq.offsets, seq.timestamps, H, dh, dh, 1e-5, workers=1)
    return float(np.sum(y * G))


@pytest.mark.parametrize("seed,lengths,affine,bias,per_head", [
    (10, [3, 5, 0, 4], True, True, True),
    (11, [7, 1], False, False, False),
])
def test_layer_gradient_matches_finite_differences(seed, lengths, affine, bias, per_head):
    # every input and parameter of one layer against a central difference of
    # L = sum(layer_fwd(...) * G); a wrong term anywhere in the chain (f2, the gate, the
    # LayerNorm backward, the attention, SiLU' or f1) fails one of these entries
    seq, w, x, G, H, dh = _layer_case(seed, lengths, affine=affine, bias=bias, per_head=per_head)
    got = bwd.layer_bwd(x, w, seq.offsets, seq.timestamps, H, dh, dh, G)
    eps = 1e-6
    targets = {"dx": ("x", x)}
    for name, field in (("dw1", "w1"), ("db1", "b1"), ("dw2", "w2"), ("db2", "b2"),
                        ("dgamma", "ln_gamma"), ("dbeta", "ln_beta"),
                        ("drab_pos", "rab_pos"), ("drab_time", "rab_time")):
        if getattr(w, field) is not None:
            targets[name] = (field, getattr(w, field))
    for gname, (field, val) in targets.items():
        num = np.zeros_like(val, dtype=np.float64)
        for idx in np.ndindex(val.shape):
            vals = []
            for sgn in (1, -1):
                pv = np.array(val, dtype=np.float64, copy=True)
                pv[idx] += sgn * eps
                if field == "x":
                    vals.append(_layer_loss(seq, w, pv, G, H, dh))
                else:
                    vals.append(_layer_loss(seq, dataclasses.replace(w, **{field: pv}), x, G, H, dh))
            num[idx] = (vals[0] - vals[1]) / (2 * eps)
        scale = max(1.0, float(np.abs(num).max()))
        np.testing.assert_allclose(got[gname], num, rtol=0, atol=5e-6 * scale, err_msg=gname)
    if not bias:  # the bias gradients are still formed: those of a zero bias
        assert got["db1"] is not None and got["db2"] is not None
    if not affine:
        assert got["dgamma"] is None and got["dbeta"] is None


def test_layer_gradient_rows_equal_the_full_gradient():
    seq, w, x, G, H, dh = _layer_case(12, [9, 0, 14, 6])
    full = bwd.layer_bwd(x, w, seq.offsets, seq.timestamps, H, dh, dh, G)
    rows = [0, 8, 9, 15, 22, 28]
    part = bwd.layer_bwd(x, w, seq.offsets, seq.timestamps, H, dh, dh, G, rows=rows)
    np.testing.assert_allclose(part["dx"][rows], full["dx"][rows], rtol=1e-12, atol=1e-12)
    mask = np.ones(x.shape[0], dtype=bool)
    mask[rows] = False
    assert np.all(part["dx"][mask] == 0) and part["dw1"] is None
