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

Parity status: pinned by central finite differences of hstu_ref.attention on small
jagged batches (tests/test_oracle_bwd.py).
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
