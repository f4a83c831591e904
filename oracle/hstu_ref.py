"""Plain fp64 CPU reference of the HSTU layer forward (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import this module.
It shares no code with the HIP library: it reads NumPy arrays produced by the seeded
input generators and computes everything itself in float64.

What it computes -- one HSTU layer, as written in "Actions Speak Louder than Words"
(chenhuiyu.github.io, "生成式推荐 16: HSTU", section "HSTU Layer 到底改了什么", the three
layer equations):

    U, V, Q, K = Split(phi1(f1(X)))                       (equation 1)
    A(X)V      = phi2(Q K^T + rab^{p,t}) V                (equation 2)
    Y          = f2(Norm(A(X)V) (.) U)                    (equation 3)

with phi1 = phi2 = SiLU and rab^{p,t} a relative bias built from the relative position
and the real time gap (same section, the sentence after the equations; also the
footnote of section 4.1 of the ltzyclt.github.io post).  The attention is pointwise:
there is no softmax or any normalisation along the sequence; LayerNorm follows the
aggregation (same page, section "不对序列做 softmax").  The batch is jagged: every
sequence is computed at its true length (same page, section "另外三块拼图", item 1).

Readings taken where the pages are silent (all listed in the design notes):
  * f1, f2 are affine maps with optional bias; weights use the "out x in" orientation,
    f1(X) = X @ w1.T + b1, f2(G) = G @ w2.T + b2.  No residual, no input norm.
  * Split order U | V | Q | K with widths H*dv, H*dv, H*dqk, H*dqk; head h owns columns
    [h*dh, (h+1)*dh) inside each block; SiLU applies to all four blocks.
  * No score scale.  Causal mask j <= i inside a sequence, diagonal included; pairs
    outside the mask contribute exactly zero.
  * rab(i, j) = P[min(i-j, P_n-1)] + T[min(T_n-1, floor(log2(1 + max(0, ts_i - ts_j))))],
    added before SiLU; tables are shared by all heads (rab_heads = 1) or per head.
  * Norm = LayerNorm over the full H*dv row, biased variance, eps, optional affine.
  * M-FALCON: every candidate of a user sits at position n_h (its history length),
    attends to all n_h history tokens and to itself only.

Parity status: every function here is pinned by tests (brute-force loops, jagged ==
per-sequence, causality, the M-FALCON reduction, closed forms and library cross-checks).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
from typing import Optional, Sequence

import numpy as np

CAUSAL = "causal"
SELF_ONLY = "self_only"

_QBLOCK = 512  # query rows per vectorised block


# ----------------------------------------------------------------------------------
# Pointwise pieces
# ----------------------------------------------------------------------------------

def silu(x: np.ndarray) -> np.ndarray:
    """SiLU(x) = x / (1 + exp(-x)) in float64 (phi1 = phi2 = SiLU)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def log2_floor_plus1(dt: np.ndarray) -> np.ndarray:
    """floor(log2(1 + dt)) for integer dt >= 0, exactly.

    1 + dt < 2^53 is an exact float64; frexp returns its binary exponent e with
    1 + dt in [2^(e-1), 2^e), so the floor of log2 is e - 1.  No float log is used.
    """
    dt = np.asarray(dt, dtype=np.int64)
    if np.any(dt < 0):
        raise ValueError("time gap must be non-negative")
    _, e = np.frexp((dt + 1).astype(np.float64))
    return e.astype(np.int64) - 1


def pos_bucket(rel: np.ndarray, n_buckets: int) -> np.ndarray:
    """Relative-position bucket min(i - j, n_buckets - 1) for i - j >= 0."""
    return np.minimum(np.asarray(rel, dtype=np.int64), n_buckets - 1)


def time_bucket(ts_q: np.ndarray, ts_k: np.ndarray, n_buckets: int) -> np.ndarray:
    """Log time-gap bucket min(n_buckets-1, floor(log2(1 + max(0, ts_q - ts_k)))), int64 gap."""
    dt = np.maximum(np.asarray(ts_q, dtype=np.int64) - np.asarray(ts_k, dtype=np.int64), 0)
    return np.minimum(log2_floor_plus1(dt), n_buckets - 1)


# ----------------------------------------------------------------------------------
# Layer pieces
# ----------------------------------------------------------------------------------

def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def f1_split(x, w1, b1, num_heads: int, dqk: int, dv: int):
    """Equation 1: Phi = SiLU(X @ w1.T + b1), split into U, V, Q, K."""
    z = _f64(x) @ _f64(w1).T
    if b1 is not None:
        z = z + _f64(b1)[None, :]
    phi = silu(z)
    hv, hq = num_heads * dv, num_heads * dqk
    u = phi[:, 0:hv]
    v = phi[:, hv:2 * hv]
    q = phi[:, 2 * hv:2 * hv + hq]
    k = phi[:, 2 * hv + hq:2 * hv + 2 * hq]
    return u, v, q, k


def _rab_row(table, h, num_heads):
    if table is None:
        return None
    t = _f64(table)
    if t.ndim == 1:
        t = t[None, :]
    if t.shape[0] == 1:
        return t[0]
    if t.shape[0] != num_heads:
        raise ValueError("rab table must have 1 or num_heads rows")
    return t[h]


def _attend_block(qh, k_all, v_all, qpos, kpos, qts, kts, allowed, ptab, ttab):
    """One block of query rows against an explicit key list (equation 2).

    qh [nq, dqk], k_all [nk, dqk], v_all [nk, dv]; qpos/qts [nq]; kpos/kts [nk];
    allowed [nq, nk] bool.  Returns [nq, dv].
    """
    s = qh @ k_all.T
    if ptab is not None:
        rel = np.maximum(qpos[:, None] - kpos[None, :], 0)  # masked pairs are dropped below
        s = s + ptab[pos_bucket(rel, ptab.shape[0])]
    if ttab is not None and qts is not None:
        s = s + ttab[time_bucket(qts[:, None], kts[None, :], ttab.shape[0])]
    a = np.where(allowed, silu(s), 0.0)
    return a @ v_all


def attention(q, k, v, offsets, timestamps, num_heads: int, dqk: int, dv: int,
              rab_pos=None, rab_time=None, *, prefix=None, mask: str = CAUSAL,
              rows: Optional[Sequence[int]] = None, workers: Optional[int] = None) -> np.ndarray:
    """Jagged pointwise aggregated attention, equation 2, fp64.

    q, k: [T][H*dqk]; v: [T][H*dv]; offsets int [B+1]; timestamps int [T] or None.
    prefix: optional (k_p [Tp][H*dqk], v_p [Tp][H*dv], offsets_p [B+1], ts_p [Tp] or None):
      per-sequence keys that precede the sequence's own tokens (an M-FALCON history).
    mask: CAUSAL -- query i (position n_p + i) sees all prefix keys and own keys j <= i;
          SELF_ONLY -- query i (position n_p) sees all prefix keys and itself only.
    rows: if given, only these global query rows are computed (others stay 0).
    Returns O [T][H*dv] (raw aggregation, before Norm).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    offsets = np.asarray(offsets, dtype=np.int64)
    ts = None if timestamps is None else np.asarray(timestamps, dtype=np.int64)
    T = q.shape[0]
    out = np.zeros((T, num_heads * dv), dtype=np.float64)
    B = offsets.shape[0] - 1
    if prefix is not None:
        kp, vp, offp, tsp = prefix
        kp, vp = _f64(kp), _f64(vp)
        offp = np.asarray(offp, dtype=np.int64)
        tsp = None if tsp is None else np.asarray(tsp, dtype=np.int64)
    use_time = rab_time is not None and ts is not None and (prefix is None or tsp is not None)

    row_sel = None
    if rows is not None:
        row_sel = np.zeros(T, dtype=bool)
        row_sel[np.asarray(rows, dtype=np.int64)] = True

    tasks = []
    for b in range(B):
        s0, s1 = int(offsets[b]), int(offsets[b + 1])
        n = s1 - s0
        if n <= 0:
            continue
        qrows = np.arange(n)
        if row_sel is not None:
            qrows = qrows[row_sel[s0:s1]]
            if qrows.size == 0:
                continue
        for h in range(num_heads):
            tasks.append((b, h, s0, n, qrows))

    def run(task):
        b, h, s0, n, qrows = task
        ptab = _rab_row(rab_pos, h, num_heads)
        ttab = _rab_row(rab_time, h, num_heads) if use_time else None
        cq = slice(h * dqk, (h + 1) * dqk)
        cv = slice(h * dv, (h + 1) * dv)
        if prefix is not None:
            p0, p1 = int(offp[b]), int(offp[b + 1])
            n_p = p1 - p0
        else:
            p0 = p1 = n_p = 0
        # key list: prefix keys then own keys
        k_own, v_own = k[s0:s0 + n, cq], v[s0:s0 + n, cv]
        if n_p > 0:
            k_all = np.concatenate([kp[p0:p1, cq], k_own])
            v_all = np.concatenate([vp[p0:p1, cv], v_own])
        else:
            k_all, v_all = k_own, v_own
        own_idx = np.arange(n)
        if mask == CAUSAL:
            kpos = np.concatenate([np.arange(n_p), n_p + own_idx])
        elif mask == SELF_ONLY:
            kpos = np.concatenate([np.arange(n_p), np.full(n, n_p)])
        else:
            raise ValueError(mask)
        if use_time:
            kts = np.concatenate([tsp[p0:p1], ts[s0:s0 + n]]) if n_p > 0 else ts[s0:s0 + n]
        else:
            kts = None
        res = []
        for c0 in range(0, qrows.size, _QBLOCK):
            qi = qrows[c0:c0 + _QBLOCK]
            qpos = (n_p + qi) if mask == CAUSAL else np.full(qi.size, n_p)
            qts = ts[s0 + qi] if use_time else None
            allowed_own = (own_idx[None, :] <= qi[:, None]) if mask == CAUSAL else \
                (own_idx[None, :] == qi[:, None])
            allowed = np.concatenate([np.ones((qi.size, n_p), dtype=bool), allowed_own], axis=1)
            o = _attend_block(q[s0 + qi, cq], k_all, v_all, qpos, kpos, qts, kts,
                              allowed, ptab, ttab)
            res.append((s0 + qi, cv, o))
        return res

    nw = workers if workers is not None else (os.cpu_count() or 1)
    if nw <= 1 or len(tasks) <= 1:
        results = map(run, tasks)
        for r in results:
            for rr, cv, o in r:
                out[rr, cv] = o
    else:
        with cf.ThreadPoolExecutor(max_workers=nw) as ex:
            for r in ex.map(run, tasks):
                for rr, cv, o in r:
                    out[rr, cv] = o
    return out


def norm_gate(o, u, gamma=None, beta=None, eps: float = 1e-5):
    """Norm(AV) (.) U: LayerNorm over each full H*dv row (biased variance), then the gate."""
    o = _f64(o)
    mu = o.mean(axis=1, keepdims=True)
    var = ((o - mu) ** 2).mean(axis=1, keepdims=True)
    nrm = (o - mu) / np.sqrt(var + eps)
    if gamma is not None:
        nrm = nrm * _f64(gamma)[None, :]
    if beta is not None:
        nrm = nrm + _f64(beta)[None, :]
    return nrm * _f64(u)


def f2(g, w2, b2=None):
    """Equation 3's output projection: Y = G @ w2.T + b2."""
    y = _f64(g) @ _f64(w2).T
    if b2 is not None:
        y = y + _f64(b2)[None, :]
    return y


# ----------------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------------

def _rows_tokens(offsets, rows):
    """Tokens of every sequence that holds one of ``rows`` (those need K and V)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    seqs = np.unique(np.searchsorted(offsets, rows, side="right") - 1)
    toks = [np.arange(offsets[b], offsets[b + 1]) for b in seqs]
    return np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)


def layer_fwd(x, weights, offsets, timestamps, num_heads: int, dqk: int, dv: int,
              eps: float = 1e-5, *, rows=None, workers=None, intermediates: bool = False):
    """One HSTU layer (equations 1-3) on a jagged batch, fp64.

    weights: object with w1, b1, w2, b2, ln_gamma, ln_beta, rab_pos, rab_time (any
    optional one may be None).  rows: if given, only these output rows are computed
    (the rest of Y is left 0); K and V are still formed for every token of the
    sequences involved.
    """
    x = _f64(x)
    T = x.shape[0]
    if rows is None:
        u, v, q, k = f1_split(x, weights.w1, weights.b1, num_heads, dqk, dv)
    else:
        toks = _rows_tokens(offsets, rows)
        hv, hq = num_heads * dv, num_heads * dqk
        u = np.zeros((T, hv)); v = np.zeros((T, hv))
        q = np.zeros((T, hq)); k = np.zeros((T, hq))
        if toks.size:
            uu, vv, qq, kk = f1_split(x[toks], weights.w1, weights.b1, num_heads, dqk, dv)
            u[toks], v[toks], q[toks], k[toks] = uu, vv, qq, kk
    o = attention(q, k, v, offsets, timestamps, num_heads, dqk, dv,
                  weights.rab_pos, weights.rab_time, rows=rows, workers=workers)
    if rows is None:
        g = norm_gate(o, u, weights.ln_gamma, weights.ln_beta, eps)
        y = f2(g, weights.w2, weights.b2)
    else:
        r = np.asarray(rows, dtype=np.int64)
        y = np.zeros((T, np.asarray(weights.w2).shape[0]))
        g = np.zeros_like(o)
        g[r] = norm_gate(o[r], u[r], weights.ln_gamma, weights.ln_beta, eps)
        y[r] = f2(g[r], weights.w2, weights.b2)
    if intermediates:
        return y, dict(u=u, v=v, q=q, k=k, o=o, g=g)
    return y


def mfalcon_fwd(x_hist, hist_offsets, hist_ts, x_cand, cand_offsets, cand_ts, weights,
                num_heads: int, dqk: int, dv: int, eps: float = 1e-5, *, workers=None):
    """M-FALCON ranking forward, fp64 (ltzyclt.github.io section 5.2; chenhuiyu.github.io
    section "另外三块拼图", item 3).

    The history pass is the plain causal layer; its K and V are computed once.  Each
    candidate of user b sits at position n_h = len(history_b), attends to all history
    tokens (relative position n_h - j, gap ts_c - ts_j) and to itself (position gap 0,
    time gap 0), never to other candidates.  Returns (y_hist, y_cand).
    """
    y_hist, mid = layer_fwd(x_hist, weights, hist_offsets, hist_ts, num_heads, dqk, dv, eps,
                            workers=workers, intermediates=True)
    u, v, q, k = f1_split(x_cand, weights.w1, weights.b1, num_heads, dqk, dv)
    o = attention(q, k, v, cand_offsets, cand_ts, num_heads, dqk, dv,
                  weights.rab_pos, weights.rab_time,
                  prefix=(mid["k"], mid["v"], hist_offsets, hist_ts), mask=SELF_ONLY,
                  workers=workers)
    g = norm_gate(o, u, weights.ln_gamma, weights.ln_beta, eps)
    return y_hist, f2(g, weights.w2, weights.b2)
