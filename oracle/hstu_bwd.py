"""Plain fp64 CPU reference of the gradients of the HSTU attention (test infrastructure only).

Only tests and the smoke check may import this module; it shares no code with the HIP
library.  It differentiates equation 2 of the layer ("Actions Speak Louder than Words" as
retold on chenhuiyu.github.io, section "HSTU Layer 到底改了什么"), the pointwise attention

    S = Q K^T + rab^{p,t},   A = SiLU(S) on allowed pairs (0 elsewhere),   O = A V,

per sequence and head under the causal mask.  With the upstream gradient dO (of the loss
with respect to O) the chain rule gives, pair by pair:

    dV = A^T dO,   dA = dO V^T,   dS = dA * SiLU'(S) on allowed pairs (0 elsewhere),
    dQ = dS K,     dK = dS^T Q,
    d rab_pos[b]  = sum of dS over the pairs whose position bucket is b,
    d rab_time[b] = sum of dS over the pairs whose time bucket is b,

with SiLU'(x) = sigma(x) (1 + x (1 - sigma(x))).  There is no softmax, so no row
statistics enter the gradient.  The pages do not discuss training-time gradients; this
is the derivative of the forward that the forward oracle (hstu_ref.attention) computes.

layer_bwd differentiates the whole layer (equations 1-3, the composition that
hstu_ref.layer_fwd computes) by the chain rule, for the upstream gradient dY:

    f2:        dG = dY w2,   dw2 = dY^T G,   db2 = sum_t dY
    gate:      dU = dG (.) N,   dN = dG (.) U
    LayerNorm: N = xhat gamma + beta, xhat = (O - mean) / sigma over each H*dv row,
               dgamma = sum_t dN (.) xhat,  dbeta = sum_t dN,  dxhat = dN gamma,
               dO = (dxhat - mean(dxhat) - xhat mean(dxhat (.) xhat)) / sigma
    attention: dQ, dK, dV, d rab from attention_bwd
    f1:        dZ = [dU | dV | dQ | dK] (.) SiLU'(Z),  Z = X w1^T + b1,
               dX = dZ w1,   dw1 = dZ^T X,   db1 = sum_t dZ

Parity status: attention_bwd and layer_bwd are pinned by central finite differences of
hstu_ref.attention and hstu_ref.layer_fwd on small jagged batches
(tests/test_oracle_bwd.py).
"""

from __future__ import annotations

import numpy as np

from . import hstu_ref as ref


def silu_grad(x: np.ndarray) -> np.ndarray:
    """d/dx [x sigma(x)] = sigma(x) (1 + x (1 - sigma(x))) in float64."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-x))
    return s * (1.0 + x * (1.0 - s))


def attention_bwd(q, k, v, d_out, offsets, timestamps, num_heads: int, dqk: int, dv: int,
                  rab_pos=None, rab_time=None, *, rows=None):
    """Gradients of hstu_ref.attention (causal, no prefix) with respect to q, k, v and the
    two bias tables, for the upstream gradient d_out [T][H*dv].

    Returns (dq [T][H*dqk], dk [T][H*dqk], dv [T][H*dv], d_rab_pos, d_rab_time); a table
    gradient has the table's shape (rows 1 or H), or is None when the table is None.
    rows: if given, only these global rows of dq, dk and dv are computed (the others stay
    0) and the table gradients are None; see _attention_bwd_rows.
    """
    if rows is not None:
        return _attention_bwd_rows(q, k, v, d_out, offsets, timestamps, num_heads, dqk, dv,
                                   rab_pos, rab_time, rows)
    q, k, v, g = (np.asarray(a, dtype=np.float64) for a in (q, k, v, d_out))
    offsets = np.asarray(offsets, dtype=np.int64)
    ts = None if timestamps is None else np.asarray(timestamps, dtype=np.int64)
    use_time = rab_time is not None and ts is not None
    dq, dk, dvv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    P = None if rab_pos is None else np.atleast_2d(np.asarray(rab_pos, dtype=np.float64))
    Tt = None if rab_time is None else np.atleast_2d(np.asarray(rab_time, dtype=np.float64))
    dP = None if P is None else np.zeros_like(P)
    dT = None if Tt is None else np.zeros_like(Tt)
    for b in range(offsets.shape[0] - 1):
        s0, s1 = int(offsets[b]), int(offsets[b + 1])
        n = s1 - s0
        if n <= 0:
            continue
        i = np.arange(n)
        allowed = i[None, :] <= i[:, None]
        pb = ref.pos_bucket(np.maximum(i[:, None] - i[None, :], 0), P.shape[1]) if P is not None else None
        tb = ref.time_bucket(ts[s0:s1][:, None], ts[s0:s1][None, :], Tt.shape[1]) if use_time else None
        for h in range(num_heads):
            cq, cv = slice(h * dqk, (h + 1) * dqk), slice(h * dv, (h + 1) * dv)
            qh, kh, vh, gh = q[s0:s1, cq], k[s0:s1, cq], v[s0:s1, cv], g[s0:s1, cv]
            s = qh @ kh.T
            rp = None if P is None else (P[0] if P.shape[0] == 1 else P[h])
            rt = None if not use_time else (Tt[0] if Tt.shape[0] == 1 else Tt[h])
            if rp is not None:
                s = s + rp[pb]
            if rt is not None:
                s = s + rt[tb]
            a = np.where(allowed, ref.silu(s), 0.0)
            da = gh @ vh.T
            ds = np.where(allowed, da * silu_grad(s), 0.0)
            dvv[s0:s1, cv] += a.T @ gh
            dq[s0:s1, cq] += ds @ kh
            dk[s0:s1, cq] += ds.T @ qh
            if rp is not None:
                row = 0 if P.shape[0] == 1 else h
                np.add.at(dP[row], pb[allowed], ds[allowed])
            if rt is not None:
                row = 0 if Tt.shape[0] == 1 else h
                np.add.at(dT[row], tb[allowed], ds[allowed])
    if dP is not None and np.ndim(rab_pos) == 1:
        dP = dP[0]
    if dT is not None and np.ndim(rab_time) == 1:
        dT = dT[0]
    return dq, dk, dvv, dP, dT


def _attention_bwd_rows(q, k, v, d_out, offsets, timestamps, num_heads, dqk, dv, rab_pos,
                        rab_time, rows):
    """The same gradients at chosen rows only, for sequences too long for the full pair
    matrices.  Row r of dq needs the pairs (r, j <= r) of its sequence; row r of dk and dv
    needs the pairs (i >= r, r).  Each is formed from its own slice of S, A and dA, with
    the same formulas as attention_bwd."""
    q, k, v, g = (np.asarray(a, dtype=np.float64) for a in (q, k, v, d_out))
    offsets = np.asarray(offsets, dtype=np.int64)
    ts = None if timestamps is None else np.asarray(timestamps, dtype=np.int64)
    use_time = rab_time is not None and ts is not None
    P = None if rab_pos is None else np.atleast_2d(np.asarray(rab_pos, dtype=np.float64))
    Tt = None if rab_time is None else np.atleast_2d(np.asarray(rab_time, dtype=np.float64))
    dq, dk, dvv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    rows = np.unique(np.asarray(rows, dtype=np.int64))
    seq_of = np.searchsorted(offsets, rows, side="right") - 1
    for b in np.unique(seq_of):
        s0, s1 = int(offsets[b]), int(offsets[b + 1])
        n = s1 - s0
        r = rows[seq_of == b] - s0          # local rows
        i = np.arange(n)

        def bias(qi, kj, h):
            # rab for the pairs (qi[:, None], kj[None, :]) of head h
            out = np.zeros((qi.size, kj.size))
            if P is not None:
                rp = P[0] if P.shape[0] == 1 else P[h]
                out += rp[ref.pos_bucket(np.maximum(qi[:, None] - kj[None, :], 0), P.shape[1])]
            if use_time:
                rt = Tt[0] if Tt.shape[0] == 1 else Tt[h]
                out += rt[ref.time_bucket(ts[s0 + qi][:, None], ts[s0 + kj][None, :], Tt.shape[1])]
            return out

        for h in range(num_heads):
            cq, cv = slice(h * dqk, (h + 1) * dqk), slice(h * dv, (h + 1) * dv)
            qh, kh, vh, gh = q[s0:s1, cq], k[s0:s1, cq], v[s0:s1, cv], g[s0:s1, cv]
            # rows as queries: pairs (r, j)
            sq = qh[r] @ kh.T + bias(r, i, h)
            ok = i[None, :] <= r[:, None]
            dsq = np.where(ok, (gh[r] @ vh.T) * silu_grad(sq), 0.0)
            dq[s0 + r, cq] = dsq @ kh
            # rows as keys: pairs (i, r)
            sk = qh @ kh[r].T + bias(i, r, h)
            ok = i[:, None] >= r[None, :]
            ak = np.where(ok, ref.silu(sk), 0.0)
            dsk = np.where(ok, (gh @ vh[r].T) * silu_grad(sk), 0.0)
            dk[s0 + r, cq] = dsk.T @ qh
            dvv[s0 + r, cv] = ak.T @ gh
    return dq, dk, dvv, None, None


def _layernorm_parts(o, eps):
    mu = o.mean(axis=1, keepdims=True)
    var = ((o - mu) ** 2).mean(axis=1, keepdims=True)
    sigma = np.sqrt(var + eps)
    return (o - mu) / sigma, sigma


def _forward_and_d_o(x, weights, offsets, ts, num_heads, dqk, dv, g_y, eps, workers):
    """The forward pieces the gradient needs and everything up to dO (the attention
    output's gradient), for every row."""
    w1, w2 = ref._f64(weights.w1), ref._f64(weights.w2)
    hv, hq = num_heads * dv, num_heads * dqk
    z = x @ w1.T
    if weights.b1 is not None:
        z = z + ref._f64(weights.b1)[None, :]
    phi = ref.silu(z)
    u, v, q, k = (phi[:, :hv], phi[:, hv:2 * hv], phi[:, 2 * hv:2 * hv + hq],
                  phi[:, 2 * hv + hq:2 * hv + 2 * hq])
    o = ref.attention(q, k, v, offsets, ts, num_heads, dqk, dv, weights.rab_pos,
                      weights.rab_time, workers=workers)
    xhat, sigma = _layernorm_parts(o, eps)
    gamma = None if weights.ln_gamma is None else ref._f64(weights.ln_gamma)
    beta = None if weights.ln_beta is None else ref._f64(weights.ln_beta)
    n = xhat * (gamma[None, :] if gamma is not None else 1.0)
    if beta is not None:
        n = n + beta[None, :]
    gate = n * u
    d_gate = g_y @ w2                       # f2
    du = d_gate * n                         # the gate
    dn = d_gate * u
    dxhat = dn * (gamma[None, :] if gamma is not None else 1.0)
    do = (dxhat - dxhat.mean(axis=1, keepdims=True)  # LayerNorm
          - xhat * (dxhat * xhat).mean(axis=1, keepdims=True)) / sigma
    return dict(z=z, u=u, v=v, q=q, k=k, xhat=xhat, gate=gate, du=du, dn=dn, do=do,
                gamma=gamma, beta=beta)


def layer_bwd(x, weights, offsets, timestamps, num_heads: int, dqk: int, dv: int, d_y,
              eps: float = 1e-5, *, rows=None, workers=None):
    """Gradients of hstu_ref.layer_fwd (causal) for the upstream gradient d_y [T][d].

    Returns a dict with dx [T][d] and the parameter gradients dw1, db1, dw2, db2, dgamma,
    dbeta, drab_pos, drab_time (dgamma / dbeta / drab_* are None when that parameter is
    None; db1 and db2 are the gradients of a bias added there, formed in any case).
    rows: if given, only these rows of dx are formed (others 0) and every parameter
    gradient is None.  The forward and dO are then formed for the whole of each sequence
    that holds one of the rows (the key-side gradients of a row need dO of every later
    query), and the attention gradient at those rows only.
    """
    x = ref._f64(x)
    g_y = ref._f64(d_y)
    w1 = ref._f64(weights.w1)
    offsets = np.asarray(offsets, dtype=np.int64)
    ts = None if timestamps is None else np.asarray(timestamps, dtype=np.int64)
    if rows is not None:
        rows = np.unique(np.asarray(rows, dtype=np.int64))
        seqs = np.unique(np.searchsorted(offsets, rows, side="right") - 1)
        dx = np.zeros_like(x)
        for b in seqs:
            s0, s1 = int(offsets[b]), int(offsets[b + 1])
            off_b = np.array([0, s1 - s0])
            ts_b = None if ts is None else ts[s0:s1]
            f = _forward_and_d_o(x[s0:s1], weights, off_b, ts_b, num_heads, dqk, dv,
                                 g_y[s0:s1], eps, workers)
            r = rows[(rows >= s0) & (rows < s1)] - s0
            dq, dk, dvv, _, _ = attention_bwd(f["q"], f["k"], f["v"], f["do"], off_b, ts_b,
                                              num_heads, dqk, dv, weights.rab_pos,
                                              weights.rab_time, rows=r)
            dz = np.concatenate([f["du"][r], dvv[r], dq[r], dk[r]], axis=1) * silu_grad(f["z"][r])
            dx[s0 + r] = dz @ w1
        return dict(dx=dx, dw1=None, db1=None, dw2=None, db2=None, dgamma=None, dbeta=None,
                    drab_pos=None, drab_time=None)
    f = _forward_and_d_o(x, weights, offsets, ts, num_heads, dqk, dv, g_y, eps,
                         1 if workers is None else workers)
    dq, dk, dvv, dP, dT = attention_bwd(f["q"], f["k"], f["v"], f["do"], offsets, ts,
                                        num_heads, dqk, dv, weights.rab_pos, weights.rab_time)
    dz = np.concatenate([f["du"], dvv, dq, dk], axis=1) * silu_grad(f["z"])  # f1 and SiLU
    return dict(dx=dz @ w1, dw1=dz.T @ x, db1=dz.sum(axis=0), dw2=g_y.T @ f["gate"],
                db2=g_y.sum(axis=0),
                dgamma=(f["dn"] * f["xhat"]).sum(axis=0) if f["gamma"] is not None else None,
                dbeta=f["dn"].sum(axis=0) if f["beta"] is not None else None,
                drab_pos=dP, drab_time=dT)
