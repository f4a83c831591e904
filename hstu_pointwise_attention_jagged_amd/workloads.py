"""Seeded synthetic inputs for the HSTU layer forward.

This module only *draws* inputs: sequence lengths, token rows, weights, timestamps,
relative-bias tables and the raw random numbers that the Stochastic Length rule
consumes.  It performs none of the layer's arithmetic (no projection, activation,
attention, normalisation or length rule), so the HIP path and the fp64 oracle can both
be fed from it without sharing any computation.

Workload shapes follow the pages' workloads:
  * sequence length 8192, embedding 1024, 24 layers -- the largest configuration
    reported in "Actions Speak Louder than Words" (chenhuiyu.github.io, section
    "实验究竟证明了什么");
  * Stochastic Length at N=4096, alpha=1.6 (same page, section "另外三块拼图", item 2);
  * 1024 candidates per user for M-FALCON (same section, item 3);
  * interleaved item/action histories (ltzyclt.github.io, section 3.2), which reach
    the kernels only as token rows.
All values are synthetic; no dataset is read.

Conventions shared by both consumers:
  * X rows, f1/f2 weights are drawn in fp32 and rounded once to bf16 (round to
    nearest even).  ``*_f32`` arrays hold the rounded values exactly; ``*_bits`` the
    raw bf16 bit patterns.
  * Weights use the "out x in" orientation: f1(X) = X @ w1.T (+ b1), w1 is
    [2H(dv+dqk)][d]; f2(G) = G @ w2.T (+ b2), w2 is [d][H*dv].
  * Timestamps are int32, start at 0 per user and grow by Geometric(p) gaps.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


# ----------------------------------------------------------------------------------
# bf16 rounding (input preparation only)
# ----------------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact fp32 value of bf16 bit patterns."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 array holding the bf16-rounded values of ``x``."""
    return bf16_to_f32(bf16_bits(x))


def round_f16(x: np.ndarray) -> np.ndarray:
    """fp32 array holding the fp16-rounded (nearest even) values of ``x``."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


# ----------------------------------------------------------------------------------
# Data classes
# ----------------------------------------------------------------------------------

@dataclasses.dataclass
class LayerDims:
    d_model: int
    num_heads: int
    dqk: int
    dv: int
    pos_buckets: int = 64
    time_buckets: int = 32
    rab_heads: int = 1
    ln_eps: float = 1e-5

    @property
    def uvqk_width(self) -> int:
        return 2 * self.num_heads * (self.dqk + self.dv)

    @property
    def hdv(self) -> int:
        return self.num_heads * self.dv


@dataclasses.dataclass
class Jagged:
    offsets: np.ndarray        # int32 [B+1]
    timestamps: np.ndarray     # int32 [T]

    @property
    def batch(self) -> int:
        return int(self.offsets.shape[0] - 1)

    @property
    def total(self) -> int:
        return int(self.offsets[-1])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.offsets.astype(np.int64))

    @property
    def max_len(self) -> int:
        return int(self.lengths.max()) if self.batch > 0 else 0


@dataclasses.dataclass
class LayerWeights:
    w1: np.ndarray                     # fp32 (bf16-exact) [2H(dv+dqk)][d]
    w2: np.ndarray                     # fp32 (bf16-exact) [d][H*dv]
    b1: Optional[np.ndarray] = None    # fp32 [2H(dv+dqk)]
    b2: Optional[np.ndarray] = None    # fp32 [d]
    ln_gamma: Optional[np.ndarray] = None  # fp32 [H*dv]
    ln_beta: Optional[np.ndarray] = None   # fp32 [H*dv]
    rab_pos: Optional[np.ndarray] = None   # fp32 [rab_heads][pos_buckets]
    rab_time: Optional[np.ndarray] = None  # fp32 [rab_heads][time_buckets]


@dataclasses.dataclass
class Workload:
    name: str
    dims: LayerDims
    seq: Jagged
    x: np.ndarray                  # fp32 (bf16-exact) [T][d]
    weights: LayerWeights
    description: str = ""
    # Stochastic Length inputs (raw batch before the length rule is applied)
    raw: Optional["RawSLBatch"] = None
    # M-FALCON candidates
    cand: Optional[Jagged] = None
    x_cand: Optional[np.ndarray] = None


@dataclasses.dataclass
class RawSLBatch:
    """A raw jagged batch plus the random numbers the Stochastic Length rule draws."""
    seq: Jagged
    x: np.ndarray                  # fp32 (bf16-exact) [T_raw][d]
    u_keep: np.ndarray             # float64 [B], uniform on [0,1)
    keys: np.ndarray               # uint32 [T_raw], i.i.d. uniform 32-bit priorities
    n_target: int = 4096
    alpha: float = 1.6


# ----------------------------------------------------------------------------------
# Draws
# ----------------------------------------------------------------------------------

def offsets_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(lengths.shape[0] + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    assert off[-1] < 2**31
    return off.astype(np.int32)


def draw_timestamps(rng: np.random.Generator, lengths, p: float = 0.01) -> np.ndarray:
    """Per user: ts_0 = 0, then strictly increasing with Geometric(p) gaps on {1,2,...}."""
    parts = []
    for n in np.asarray(lengths, dtype=np.int64):
        if n == 0:
            continue
        gaps = rng.geometric(p, size=int(n) - 1)
        ts = np.concatenate([[0], np.cumsum(gaps)])
        parts.append(ts)
    if not parts:
        return np.zeros(0, dtype=np.int32)
    ts = np.concatenate(parts)
    assert ts.max() < 2**31
    return ts.astype(np.int32)


def draw_x(rng: np.random.Generator, total: int, d: int) -> np.ndarray:
    return round_bf16(rng.standard_normal((total, d), dtype=np.float32))


def draw_attention_grad_inputs(rng: np.random.Generator, total: int, width: int):
    """Inputs of the attention gradient: Q, K, V as fp16 values (float32 arrays holding
    fp16-exact numbers) drawn N(0.2, 0.6^2), the mean and spread of the projected and
    activated rows the forward attends over (scores of mean about 5 and spread about 4.5
    at 128 features), and the upstream gradient dO drawn N(0, 1) in float32."""
    q, k, v = (round_f16(np.float32(0.2) + np.float32(0.6) *
                         rng.standard_normal((total, width), dtype=np.float32)) for _ in range(3))
    g = rng.standard_normal((total, width), dtype=np.float32)
    return q, k, v, g


def draw_weights(rng: np.random.Generator, dims: LayerDims, *, bias: bool = False,
                 affine: bool = False, rab: bool = True, rab_std: float = 0.02) -> LayerWeights:
    d, h = dims.d_model, dims.num_heads
    n1 = dims.uvqk_width
    hdv = dims.hdv
    w1 = round_bf16((rng.standard_normal((n1, d), dtype=np.float32) / np.float32(np.sqrt(d))))
    w2 = round_bf16((rng.standard_normal((d, hdv), dtype=np.float32) / np.float32(np.sqrt(hdv))))
    w = LayerWeights(w1=w1, w2=w2)
    if bias:
        w.b1 = (0.1 * rng.standard_normal(n1)).astype(np.float32)
        w.b2 = (0.1 * rng.standard_normal(d)).astype(np.float32)
    if affine:
        w.ln_gamma = (1.0 + 0.1 * rng.standard_normal(hdv)).astype(np.float32)
        w.ln_beta = (0.1 * rng.standard_normal(hdv)).astype(np.float32)
    if rab:
        w.rab_pos = (rab_std * rng.standard_normal((dims.rab_heads, dims.pos_buckets))).astype(np.float32)
        w.rab_time = (rab_std * rng.standard_normal((dims.rab_heads, dims.time_buckets))).astype(np.float32)
    return w


def zipf_lengths(rng: np.random.Generator, count: int, s: float, lo: int, hi: int) -> np.ndarray:
    """Truncated Zipf: P(k) proportional to k^-s on the integers [lo, hi]."""
    k = np.arange(lo, hi + 1, dtype=np.float64)
    p = k ** (-s)
    p /= p.sum()
    return rng.choice(np.arange(lo, hi + 1), size=count, p=p).astype(np.int64)


def loguniform_lengths(rng: np.random.Generator, count: int, lo: int, hi: int) -> np.ndarray:
    u = rng.random(count)
    n = np.floor(lo * (hi / lo) ** u).astype(np.int64)
    return np.clip(n, lo, hi)


def jagged_from_lengths(rng: np.random.Generator, lengths) -> Jagged:
    lengths = np.asarray(lengths, dtype=np.int64)
    return Jagged(offsets=offsets_from_lengths(lengths), timestamps=draw_timestamps(rng, lengths))


def random_layer(seed: int, lengths, dims: LayerDims, **wkw) -> Workload:
    """A small custom workload (used by tests)."""
    rng = np.random.default_rng(seed)
    seq = jagged_from_lengths(rng, lengths)
    x = draw_x(rng, seq.total, dims.d_model)
    w = draw_weights(rng, dims, **wkw)
    return Workload(name=f"custom-{seed}", dims=dims, seq=seq, x=x, weights=w)


# ----------------------------------------------------------------------------------
# Named workloads
# ----------------------------------------------------------------------------------

CONFIG_NAMES = {
    0: "tiny-4seq-d64",
    1: "zipf64-d256-h4x64",
    2: "uniform8x8192-d1024-h8x128",
    3: "stochastic-length128-d512-h8x64",
    4: "mfalcon16x(4096+1024)-d512-h8x64",
}


def config(idx: int, seed: Optional[int] = None, *, batch: Optional[int] = None,
           seq_len: Optional[int] = None) -> Workload:
    """Named synthetic workloads.

    0  tiny: lengths {5,17,32,64}, d=64, 2 heads of 32.
    1  64 users, truncated Zipf(1.2) lengths on [16,1024], d=256, 4 heads of 64.
    2  8 users x 8192 tokens, d=1024, 8 heads of 128 (``batch``/``seq_len`` may shrink it).
    3  128 users, raw lengths log-uniform on [256,4096] plus the Stochastic Length
       randomness (N=4096, alpha=1.6); d=512, 8 heads of 64.  ``seq``/``x`` hold the
       raw batch; the length rule itself is applied by its consumer.
    4  16 users x 4096-token history + 1024 candidates, d=512, 8 heads of 64.
    """
    seed = idx if seed is None else seed
    rng = np.random.default_rng(seed)
    if idx == 0:
        dims = LayerDims(d_model=64, num_heads=2, dqk=32, dv=32)
        lengths = np.array([5, 17, 32, 64])
    elif idx == 1:
        dims = LayerDims(d_model=256, num_heads=4, dqk=64, dv=64)
        lengths = zipf_lengths(rng, batch or 64, 1.2, 16, 1024)
    elif idx == 2:
        dims = LayerDims(d_model=1024, num_heads=8, dqk=128, dv=128)
        lengths = np.full(batch or 8, seq_len or 8192)
    elif idx == 3:
        dims = LayerDims(d_model=512, num_heads=8, dqk=64, dv=64)
        lengths = loguniform_lengths(rng, batch or 128, 256, 4096)
    elif idx == 4:
        dims = LayerDims(d_model=512, num_heads=8, dqk=64, dv=64)
        lengths = np.full(batch or 16, seq_len or 4096)
    else:
        raise ValueError(f"unknown config {idx}")

    seq = jagged_from_lengths(rng, lengths)
    x = draw_x(rng, seq.total, dims.d_model)
    w = draw_weights(rng, dims)
    wl = Workload(name=CONFIG_NAMES[idx], dims=dims, seq=seq, x=x, weights=w,
                  description=config.__doc__ or "")
    if idx == 3:
        raw = RawSLBatch(seq=seq, x=x, u_keep=rng.random(seq.batch),
                         keys=rng.integers(0, 2**32, size=seq.total, dtype=np.uint64).astype(np.uint32))
        wl.raw = raw
    if idx == 4:
        n_cand = 1024 if batch is None and seq_len is None else max(1, (seq_len or 4096) // 4)
        b = seq.batch
        c_len = np.full(b, n_cand, dtype=np.int64)
        last = seq.timestamps[seq.offsets[1:] - 1].astype(np.int64)
        req = last + rng.geometric(0.01, size=b)
        cts = np.repeat(req, c_len).astype(np.int32)
        wl.cand = Jagged(offsets=offsets_from_lengths(c_len), timestamps=cts)
        wl.x_cand = draw_x(rng, int(c_len.sum()), dims.d_model)
    return wl
