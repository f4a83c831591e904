"""Scalar triple-loop HSTU layer, for tiny inputs only (test infrastructure only).

A second, deliberately naive statement of the same layer as ``hstu_ref`` -- pure Python
floats and ints, one pair (i, j) at a time, every sum written out -- so the vectorised
reference can be checked against it element by element.  It follows the same page
passages: "Actions Speak Louder than Words" (chenhuiyu.github.io, section "HSTU Layer
到底改了什么", equations 1-3; section "不对序列做 softmax"), with the same readings
for the unstated details (see ``hstu_ref``).  The log time bucket uses
``int.bit_length`` rather than any float logarithm.
"""

from __future__ import annotations

import math


def _silu(x: float) -> float:
    if x < -700.0:
        return 0.0 * x
    return x / (1.0 + math.exp(-x))


def _bucket_time(ts_q: int, ts_k: int, n_buckets: int) -> int:
    dt = ts_q - ts_k
    if dt < 0:
        dt = 0
    return min((dt + 1).bit_length() - 1, n_buckets - 1)


def _table(t, h):
    if t is None:
        return None
    rows = [list(map(float, r)) for r in (t if hasattr(t[0], "__len__") else [t])]
    return rows[h] if len(rows) > 1 else rows[0]


def layer_fwd(x, w, offsets, timestamps, H, dqk, dv, eps=1e-5, *, intermediates=False):
    """Plain loops over tokens, heads, query i and key j <= i."""
    X = [list(map(float, r)) for r in x]
    T = len(X)
    d = len(X[0]) if T else 0
    W1 = [list(map(float, r)) for r in w.w1]
    N1 = len(W1)
    b1 = [0.0] * N1 if w.b1 is None else list(map(float, w.b1))
    # f1 + SiLU
    phi = []
    for t in range(T):
        row = []
        for c in range(N1):
            acc = b1[c]
            for e in range(d):
                acc += X[t][e] * W1[c][e]
            row.append(_silu(acc))
        phi.append(row)
    hv, hq = H * dv, H * dqk
    U = [r[0:hv] for r in phi]
    V = [r[hv:2 * hv] for r in phi]
    Q = [r[2 * hv:2 * hv + hq] for r in phi]
    K = [r[2 * hv + hq:2 * hv + 2 * hq] for r in phi]
    ts = None if timestamps is None else [int(t) for t in timestamps]

    O = [[0.0] * hv for _ in range(T)]
    B = len(offsets) - 1
    for b in range(B):
        s0, s1 = int(offsets[b]), int(offsets[b + 1])
        for h in range(H):
            P = _table(w.rab_pos, h)
            TT = _table(w.rab_time, h) if ts is not None else None
            for i in range(s1 - s0):
                for j in range(i + 1):
                    s = 0.0
                    for e in range(dqk):
                        s += Q[s0 + i][h * dqk + e] * K[s0 + j][h * dqk + e]
                    if P is not None:
                        s += P[min(i - j, len(P) - 1)]
                    if TT is not None:
                        s += TT[_bucket_time(ts[s0 + i], ts[s0 + j], len(TT))]
                    a = _silu(s)
                    for e in range(dv):
                        O[s0 + i][h * dv + e] += a * V[s0 + j][h * dv + e]
    gam = None if w.ln_gamma is None else list(map(float, w.ln_gamma))
    bet = None if w.ln_beta is None else list(map(float, w.ln_beta))
    G = []
    for t in range(T):
        row = O[t]
        mu = sum(row) / hv
        var = sum((z - mu) * (z - mu) for z in row) / hv
        inv = 1.0 / math.sqrt(var + eps)
        g = []
        for e in range(hv):
            n = (row[e] - mu) * inv
            if gam is not None:
                n *= gam[e]
            if bet is not None:
                n += bet[e]
            g.append(n * U[t][e])
        G.append(g)
    W2 = [list(map(float, r)) for r in w.w2]
    b2 = [0.0] * len(W2) if w.b2 is None else list(map(float, w.b2))
    Y = []
    for t in range(T):
        Y.append([b2[c] + sum(G[t][e] * W2[c][e] for e in range(hv)) for c in range(len(W2))])
    if intermediates:
        return Y, dict(u=U, v=V, q=Q, k=K, o=O, g=G)
    return Y
