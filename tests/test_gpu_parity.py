"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bars (from the layer's contract): bf16 layer outputs within max-abs 2e-2 and mean-abs
2e-3 of the oracle; the raw fp32 attention output within the same bounds after dividing
by the oracle's row standard deviation; integer paths (offsets, masks, rab indices)
bit-exact, checked by decodable probes whose every (i, j) entry must recover the
oracle's table index exactly and whose masked entries must be exactly 0.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from hstu_pointwise_attention_jagged_amd import device as dev  # noqa: E402
from hstu_pointwise_attention_jagged_amd import ops  # noqa: E402
from hstu_pointwise_attention_jagged_amd import workloads as wl  # noqa: E402
from oracle import hstu_ref as ref  # noqa: E402
from oracle import stochastic_length as sl  # noqa: E402

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from hstu_pointwise_attention_jagged_amd import _lib
    _lib.load()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------------

def _layer_check(w, *, rows=None, tag=""):
    d = w.dims
    say(f"[layer] {tag} {w.name} B={w.seq.batch} T={w.seq.total} d={d.d_model} H={d.num_heads} dh={d.dqk}")
    y, uvqk = ops.hstu_layer_fwd(dev.dims_of(d), dev.weights_of(w.weights), dev.jagged_of(w.seq),
                                 dev.bf16_tensor(w.x))
    torch.cuda.synchronize()
    got = dev.bf16_to_numpy(y).astype(np.float64)
    want = ref.layer_fwd(w.x, w.weights, w.seq.offsets, w.seq.timestamps, d.num_heads, d.dqk,
                         d.dv, d.ln_eps, rows=rows)
    if rows is not None:
        got, want = got[rows], want[rows]
    err = np.abs(got - want)
    say(f"        max_abs={err.max():.3e} mean_abs={err.mean():.3e}")
    assert np.all(np.isfinite(got))
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS
    return y, uvqk


def _attn_inputs(seed, lengths, H, dh, *, ts_scale=1):
    rng = np.random.default_rng(seed)
    seq = wl.jagged_from_lengths(rng, lengths)
    if ts_scale != 1:
        seq.timestamps = (seq.timestamps.astype(np.int64) * ts_scale).astype(np.int32)
    T = seq.total
    q, k, v = (wl.round_f16(rng.standard_normal((T, H * dh), dtype=np.float32)) for _ in range(3))
    P = (0.5 * rng.standard_normal((1, 64))).astype(np.float32)
    Tt = (0.5 * rng.standard_normal((1, 32))).astype(np.float32)
    return seq, q, k, v, P, Tt


def _attn_gpu(seq, q, k, v, H, dh, P, Tt, *, prefix=None, mask="causal", with_time=True):
    dims = ops.LayerDims(d_model=max(64, H * dh), num_heads=H, dqk=dh, dv=dh,
                         pos_buckets=P.shape[1] if P is not None else 64,
                         time_buckets=Tt.shape[1] if Tt is not None else 32,
                         rab_heads=P.shape[0] if P is not None else 1)
    qkv = np.concatenate([q, k, v], axis=1)
    buf = dev.f16_tensor(qkv)
    hq = H * dh
    pref = None
    if prefix is not None:
        pseq, kp, vp = prefix
        # prefix rows share the candidates' row pitch (3 H dh: K, V, unused)
        pbuf = dev.f16_tensor(np.concatenate([kp, vp, np.zeros_like(kp)], axis=1))
        pref = (dev.jagged_of(pseq, with_time=with_time), pbuf[:, :hq], pbuf[:, hq:], pbuf.stride(0))
    out = ops.hstu_attn_fwd(dims, dev.jagged_of(seq, with_time=with_time), buf[:, :hq],
                            buf[:, hq:2 * hq], buf[:, 2 * hq:], row_stride=buf.stride(0),
                            rab_pos=dev.f32_tensor(P), rab_time=dev.f32_tensor(Tt), prefix=pref,
                            mask=mask)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _rel_err(got, want, n_keys=None, vmax=None):
    """|got - want| over the oracle's row std, with an absolute floor for fp16 A.

    A is an fp16 MFMA operand: a term whose SiLU value lies below the fp16 subnormal
    quantum (2^-24) cannot be represented, so each contributing key may be off by up to
    2^-24 * max|v| in absolute terms.  The floor only matters on rows whose every score
    is very negative (their output is ~1e-9 of a normal row's).
    """
    scale = want.std(axis=1, keepdims=True)
    if n_keys is not None:
        scale = scale + np.asarray(n_keys, dtype=np.float64)[:, None] * 2.0**-24 * vmax / MAX_ABS
    return np.abs(got - want) / np.maximum(scale, 1e-30)


def _causal_keys(seq):
    return np.concatenate([np.arange(1, n + 1) for n in seq.lengths]) if seq.total else np.zeros(0)


# ----------------------------------------------------------------------------------
# attention alone
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("H,dh,lengths", [
    (2, 32, [5, 17, 32, 64]),
    (2, 64, [0, 1, 130, 0, 257, 63, 64, 65]),
    (2, 128, [1, 300, 129, 700]),
    (1, 128, [2000]),
])
def test_attention_causal_matches_oracle(H, dh, lengths):
    say(f"[attn] causal H={H} dh={dh} lengths={lengths}")
    seq, q, k, v, P, Tt = _attn_inputs(40 + dh, lengths, H, dh)
    got = _attn_gpu(seq, q, k, v, H, dh, P, Tt)
    want = ref.attention(q, k, v, seq.offsets, seq.timestamps, H, dh, dh, P, Tt)
    e = _rel_err(got, want, _causal_keys(seq), np.abs(v).max())
    say(f"        max_rel={e.max():.3e} mean_rel={e.mean():.3e}")
    assert e.max() <= MAX_ABS and e.mean() <= MEAN_ABS


def test_attention_per_head_tables_and_no_time():
    H, dh = 4, 64
    seq, q, k, v, _, _ = _attn_inputs(51, [33, 90, 0, 200], H, dh)
    rng = np.random.default_rng(5)
    P = (0.5 * rng.standard_normal((H, 48))).astype(np.float32)
    Tt = (0.5 * rng.standard_normal((H, 20))).astype(np.float32)
    say("[attn] per-head tables")
    got = _attn_gpu(seq, q, k, v, H, dh, P, Tt)
    want = ref.attention(q, k, v, seq.offsets, seq.timestamps, H, dh, dh, P, Tt)
    assert _rel_err(got, want, _causal_keys(seq), np.abs(v).max()).max() <= MAX_ABS
    say("[attn] no timestamps")
    got = _attn_gpu(seq, q, k, v, H, dh, P, Tt, with_time=False)
    want = ref.attention(q, k, v, seq.offsets, None, H, dh, dh, P, None)
    assert _rel_err(got, want, _causal_keys(seq), np.abs(v).max()).max() <= MAX_ABS


def test_attention_self_only_with_prefix_matches_oracle():
    H, dh = 2, 64
    rng = np.random.default_rng(61)
    n_h, n_c = [100, 0, 257, 64], [7, 3, 130, 1]
    hist = wl.jagged_from_lengths(rng, n_h)
    T_h = hist.total
    kp, vp = (wl.round_f16(rng.standard_normal((T_h, H * dh), dtype=np.float32)) for _ in range(2))
    seq, q, k, v, P, Tt = _attn_inputs(62, n_c, H, dh)
    # candidates ask at a request time after the user's history
    last = np.array([hist.timestamps[hist.offsets[b + 1] - 1] if n_h[b] else 0 for b in range(4)])
    seq.timestamps = np.repeat(last + 50, n_c).astype(np.int32)
    say("[attn] self-only + prefix")
    got = _attn_gpu(seq, q, k, v, H, dh, P, Tt, prefix=(hist, kp, vp), mask="self_only")
    want = ref.attention(q, k, v, seq.offsets, seq.timestamps, H, dh, dh, P, Tt,
                         prefix=(kp, vp, hist.offsets, hist.timestamps), mask=ref.SELF_ONLY)
    n_keys = np.repeat(np.array(n_h) + 1, n_c)
    e = _rel_err(got, want, n_keys, max(np.abs(v).max(), np.abs(vp).max()))
    say(f"        max_rel={e.max():.3e} mean_rel={e.mean():.3e}")
    assert e.max() <= MAX_ABS and e.mean() <= MEAN_ABS


@pytest.mark.parametrize("dh,n_h,n_c", [
    (64, [100, 0, 257, 64], [7, 3, 130, 1]),
    (128, [0, 300, 2100, 33], [64, 129, 200, 0]),
])
def test_attention_causal_with_prefix_matches_oracle(dh, n_h, n_c):
    """Causal mask with a prefix: query i sits at position n_p + i, sees every prefix key
    and its own keys j <= i (timestamps increase from the prefix into the own rows)."""
    H = 2
    rng = np.random.default_rng(63 + dh)
    hist = wl.jagged_from_lengths(rng, n_h)
    kp, vp = (wl.round_f16(rng.standard_normal((hist.total, H * dh), dtype=np.float32)) for _ in range(2))
    seq, q, k, v, P, Tt = _attn_inputs(64 + dh, n_c, H, dh)
    last = np.array([hist.timestamps[hist.offsets[b + 1] - 1] if n_h[b] else 0 for b in range(len(n_h))])
    seq.timestamps = (seq.timestamps + np.repeat(last + 1, n_c)).astype(np.int32)
    say(f"[attn] causal + prefix dh={dh} prefix={n_h} own={n_c}")
    got = _attn_gpu(seq, q, k, v, H, dh, P, Tt, prefix=(hist, kp, vp), mask="causal")
    want = ref.attention(q, k, v, seq.offsets, seq.timestamps, H, dh, dh, P, Tt,
                         prefix=(kp, vp, hist.offsets, hist.timestamps), mask=ref.CAUSAL)
    n_keys = np.concatenate([n_h[b] + np.arange(1, n_c[b] + 1) for b in range(len(n_c))])
    e = _rel_err(got, want, n_keys, max(np.abs(v).max(), np.abs(vp).max()))
    say(f"        max_rel={e.max():.3e} mean_rel={e.mean():.3e}")
    assert e.max() <= MAX_ABS and e.mean() <= MEAN_ABS


# ----------------------------------------------------------------------------------
# bit-exact integer paths: decodable probes
# ----------------------------------------------------------------------------------

def _decode(values, table):
    cand = ref.silu(np.asarray(table, dtype=np.float64))
    return np.abs(values[..., None] - cand).argmin(axis=-1)


def _probe(lengths, *, kind, dh=128, seed=0, prefix_lengths=None, prefix_mask="self_only"):
    """Q = K = 0, V one-hot over key index (mod dh): out = SiLU(rab) exactly on allowed pairs."""
    rng = np.random.default_rng(seed)
    H = 1
    seq = wl.jagged_from_lengths(rng, lengths)
    # wide, unsorted timestamps: gaps of any size and sign, up to the int32 range
    seq.timestamps = rng.integers(-2**31, 2**31, size=seq.total, dtype=np.int64).astype(np.int32)
    if kind == "pos":
        P = (1.0 + np.arange(64) / 8.0)[None].astype(np.float32)
        Tt = None
    else:
        P = None
        Tt = (1.0 + np.arange(32) / 4.0)[None].astype(np.float32)
        # a dense band of small gaps too
        for b in range(seq.batch):
            s0, s1 = seq.offsets[b], seq.offsets[b + 1]
            if s1 - s0 > 4 and b % 2 == 0:
                seq.timestamps[s0:s1] = np.cumsum(rng.integers(0, 40, size=s1 - s0)).astype(np.int32)
    T = seq.total
    q = np.zeros((T, dh), np.float32)
    k = np.zeros((T, dh), np.float32)
    v = np.zeros((T, dh), np.float32)
    # own keys one-hot on columns base + i; prefix keys (if any) on columns j < base
    base = 64 if prefix_lengths is not None else 0
    for b in range(seq.batch):
        s0, s1 = seq.offsets[b], seq.offsets[b + 1]
        v[s0 + np.arange(s1 - s0), (base + np.arange(s1 - s0)) % dh] = 1.0
    prefix = None
    pre_ref = None
    mask = "causal"
    if prefix_lengths is not None:
        hist = wl.jagged_from_lengths(rng, prefix_lengths)
        hist.timestamps = rng.integers(-2**31, 2**31, size=hist.total, dtype=np.int64).astype(np.int32)
        kp = np.zeros((hist.total, dh), np.float32)
        vp = np.zeros((hist.total, dh), np.float32)
        for b in range(hist.batch):
            s0, s1 = hist.offsets[b], hist.offsets[b + 1]
            vp[s0 + np.arange(s1 - s0), np.arange(s1 - s0) % dh] = 1.0
        prefix = (hist, kp, vp)
        pre_ref = (kp, vp, hist.offsets, hist.timestamps)
        mask = prefix_mask
    got = _attn_gpu(seq, q, k, v, H, dh, P, Tt, prefix=prefix, mask=mask)
    want = ref.attention(q, k, v, seq.offsets, seq.timestamps, H, dh, dh, P, Tt, prefix=pre_ref,
                         mask=ref.SELF_ONLY if mask == "self_only" else ref.CAUSAL)
    return got, want, (P if kind == "pos" else Tt)[0]


@pytest.mark.parametrize("kind", ["pos", "time"])
@pytest.mark.parametrize("lengths", [[5, 17, 32, 64], [0, 1, 128, 0, 100, 127, 3]])
def test_probe_rab_indices_bit_exact(kind, lengths):
    say(f"[probe] {kind} lengths={lengths}")
    got, want, table = _probe(lengths, kind=kind, seed=len(lengths))
    zero = want == 0.0
    assert np.all(got[zero] == 0.0), "masked pairs must be exactly zero"
    nz = ~zero
    np.testing.assert_array_equal(_decode(got[nz], table), _decode(want[nz], table))


@pytest.mark.parametrize("mask", ["self_only", "causal"])
@pytest.mark.parametrize("kind", ["pos", "time"])
def test_probe_prefix_indices_bit_exact(kind, mask):
    say(f"[probe] prefix {mask} {kind}")
    got, want, table = _probe([3, 60, 1, 0], kind=kind, seed=9, prefix_lengths=[40, 64, 0, 20],
                              prefix_mask=mask)
    zero = want == 0.0
    assert np.all(got[zero] == 0.0)
    np.testing.assert_array_equal(_decode(got[~zero], table), _decode(want[~zero], table))


def test_attention_weights_saturate_past_fp16_range():
    """A = SiLU(score) travels to the P.V product as fp16 in the scaled domain A / -ln 2, so
    a weight above 65504 ln 2 (about 45403) saturates there instead of overflowing to
    infinity.  Probe: q_i, k_j on one coordinate with scores up to 9e4, V one-hot over keys,
    no bias: out[i][j] is the weight of pair (i, j) alone."""
    n, dh = 64, 64
    a = wl.round_f16(np.linspace(1.0, 300.0, n).astype(np.float32))
    q = np.zeros((n, dh), np.float32)
    k = np.zeros((n, dh), np.float32)
    v = np.zeros((n, dh), np.float32)
    q[:, 0] = a
    k[:, 0] = a[::-1]
    v[np.arange(n), np.arange(n)] = 1.0
    seq = wl.Jagged(offsets=np.array([0, n], np.int32), timestamps=np.arange(n, dtype=np.int32))
    got = _attn_gpu(seq, q, k, v, 1, dh, None, None)
    s = np.outer(a.astype(np.float64), a[::-1].astype(np.float64))
    silu = ref.silu(s)
    allowed = np.tril(np.ones((n, n), bool))
    cap = 65504.0 * np.log(2.0)
    say(f"[attn] saturation: max SiLU {silu[allowed].max():.4g}, cap {cap:.6g}")
    assert np.all(np.isfinite(got))
    assert np.all(got[~allowed] == 0.0)
    big = allowed & (silu > 1.02 * cap)
    small = allowed & (silu < 0.98 * cap)
    assert big.sum() > 100 and small.sum() > 100
    np.testing.assert_allclose(got[big], cap, rtol=1e-6)
    np.testing.assert_allclose(got[small], silu[small], rtol=2e-3)


def test_layer_with_large_weights_stays_finite():
    """f1 weights 2e4 times larger than N(0, 1/d): the f1 outputs pass the fp16 range and
    every score the fp16 limit of A; both saturate, so every output row stays finite (and
    repeats bit for bit)."""
    dims = wl.LayerDims(d_model=128, num_heads=2, dqk=64, dv=64)
    w = wl.random_layer(8, [5, 300, 129], dims)
    w.weights.w1 = wl.round_bf16((2e4 * w.weights.w1).astype(np.float32))
    d = w.dims
    args = (dev.dims_of(d), dev.weights_of(w.weights), dev.jagged_of(w.seq), dev.bf16_tensor(w.x))
    say("[layer] large weights")
    y1, u1 = ops.hstu_layer_fwd(*args)
    y2, _ = ops.hstu_layer_fwd(*args)
    torch.cuda.synchronize()
    assert float(u1.float().abs().max()) == 65504.0
    assert torch.isfinite(y1.float()).all()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# ----------------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------------

def test_layer_tiny_config():
    _layer_check(wl.config(0))


def test_layer_tiny_with_bias_affine_per_head_rab():
    w = wl.config(0)
    d = w.dims
    d.rab_heads = d.num_heads
    w.weights = wl.draw_weights(np.random.default_rng(3), d, bias=True, affine=True, rab_std=0.3)
    _layer_check(w, tag="bias+affine+per-head-rab")


def test_layer_ragged_with_empty_sequences():
    dims = wl.LayerDims(d_model=128, num_heads=2, dqk=64, dv=64)
    _layer_check(wl.random_layer(5, [0, 1, 127, 128, 129, 0, 300, 2], dims, bias=True), tag="ragged")


@pytest.mark.parametrize("heads,dh,affine", [
    (16, 32, False),  # the most heads of the LDS coefficient table; two heads per 64 features
    (3, 64, True),    # an odd head count, with gamma and beta
    (18, 32, True),   # more heads than the table holds: per-chunk statistics
    (24, 64, False),
])
def test_layer_head_counts(heads, dh, affine):
    """The f2 kernel takes a row's LayerNorm from its heads' statistics, from an LDS table
    of per-head coefficients (up to 16 heads) or per staged chunk (more heads); two row
    tiles, the second ragged."""
    dims = wl.LayerDims(d_model=128, num_heads=heads, dqk=dh, dv=dh)
    _layer_check(wl.random_layer(11 + heads, [300, 5, 129], dims, affine=affine),
                 tag=f"heads={heads} dh={dh} affine={affine}")


@pytest.mark.parametrize("keep", ["gamma", "beta"])
@pytest.mark.parametrize("lengths", [[5, 17, 32, 64], [300, 5, 129]])
def test_layer_gamma_or_beta_alone(keep, lengths):
    """LayerNorm with only gamma or only beta (the other 1 or 0): the f2 operand conversion
    runs after the small-tile f1 (first batch, 118 rows) or in the tail of the large-tile f1
    launch (second, 434 rows)."""
    dims = wl.LayerDims(d_model=128, num_heads=2, dqk=64, dv=64)
    w = wl.random_layer(21, lengths, dims, affine=True)
    if keep == "gamma":
        w.weights.ln_beta = None
    else:
        w.weights.ln_gamma = None
    _layer_check(w, tag=f"{keep} only")


def test_layer_zipf_config():
    _layer_check(wl.config(1))


def test_layer_long_uniform_config_sampled_rows():
    """Every one of the 8 sequences: the first and last row of five 128-row query tiles
    (the first two, one in the middle, the last two) plus one random row."""
    w = wl.config(2)
    rng = np.random.default_rng(0)
    off = w.seq.offsets
    rows = set()
    for b in range(w.seq.batch):
        for t in (0, 1, 31 + b, 62, 63):
            rows |= {int(off[b] + 128 * t), int(off[b] + 128 * t + 127)}
        rows.add(int(off[b] + rng.integers(0, 8192)))
    _layer_check(w, rows=sorted(rows), tag="full size, sampled rows of every sequence")


def test_layer_stochastic_length_batch_sampled_rows():
    w = wl.config(3)
    kept, new_off = sl.select(w.raw.seq.offsets, w.raw.u_keep, w.raw.keys, w.raw.n_target, w.raw.alpha)
    w.seq = wl.Jagged(offsets=new_off, timestamps=w.raw.seq.timestamps[kept])
    w.x = w.raw.x[kept]
    lens = np.diff(new_off)
    say(f"[sl] kept T={new_off[-1]} of {w.raw.seq.total}; full users={int(np.sum(lens > 776))}")
    # every kept user: its first and last row and one row in between; the longest user
    # also at every 128-row tile boundary
    rng = np.random.default_rng(3)
    rows = set()
    for b in range(len(lens)):
        if lens[b] == 0:
            continue
        a, e = int(new_off[b]), int(new_off[b + 1])
        rows |= {a, e - 1, int(a + rng.integers(0, e - a))}
    b_long = int(np.argmax(lens))
    for t in range(0, int(lens[b_long]), 128):
        rows |= {int(new_off[b_long] + t), int(min(new_off[b_long] + t + 127, new_off[b_long + 1] - 1))}
    _layer_check(w, rows=sorted(rows), tag=f"stochastic length, {len(rows)} rows of every kept user")


def test_layer_deterministic_and_guard_band():
    w = wl.config(1, batch=16)
    d = w.dims
    T = w.seq.total
    dims, wts, seq = dev.dims_of(d), dev.weights_of(w.weights), dev.jagged_of(w.seq)
    x = dev.bf16_tensor(w.x)
    big = torch.full((T + 64, d.d_model), 7.0, dtype=torch.bfloat16, device="cuda")
    ubig = torch.full((T + 64, d.uvqk_width), 7.0, dtype=torch.float16, device="cuda")
    say("[layer] determinism + guard band")
    ops.hstu_layer_fwd(dims, wts, seq, x, y=big[:T], uvqk=ubig[:T])
    y1 = big[:T].clone()
    ops.hstu_layer_fwd(dims, wts, seq, x, y=big[:T], uvqk=ubig[:T])
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), big[:T].view(torch.int16))
    assert torch.all(big[T:] == 7.0) and torch.all(ubig[T:] == 7.0)


def test_validate_jagged():
    good = wl.jagged_from_lengths(np.random.default_rng(1), [3, 0, 9])
    j = dev.jagged_of(good)
    assert ops.hstu_validate_jagged(j)
    bad = dev.jagged_of(good)
    bad.offsets = dev.i32_tensor(np.array([0, 3, 2, 12]))
    assert not ops.hstu_validate_jagged(bad)
    short = dev.jagged_of(good)
    short.max_seq_len = 5
    assert not ops.hstu_validate_jagged(short)
    cap = dev.jagged_of(good)  # total_tokens as a capacity above off[B]
    cap.total_tokens = 40
    assert ops.hstu_validate_jagged(cap)
    under = dev.jagged_of(good)
    under.total_tokens = 11
    assert not ops.hstu_validate_jagged(under)


# ----------------------------------------------------------------------------------
# M-FALCON
# ----------------------------------------------------------------------------------

def _mfalcon(w, cand, xc, bm):
    """History pass once, then candidates in micro-batches of bm per user."""
    d = w.dims
    dims, wts = dev.dims_of(d), dev.weights_of(w.weights)
    hist = dev.jagged_of(w.seq)
    y_h, uvqk_h = ops.hstu_layer_fwd(dims, wts, hist, dev.bf16_tensor(w.x))
    n_c = np.diff(cand.offsets.astype(np.int64))
    assert np.all(n_c == n_c[0])
    outs = np.zeros((cand.total, d.d_model), np.float32)
    for start in range(0, int(n_c[0]), bm):
        m = min(bm, int(n_c[0]) - start)
        sel = np.concatenate([cand.offsets[b] + start + np.arange(m) for b in range(cand.batch)])
        mc = wl.Jagged(offsets=wl.offsets_from_lengths(np.full(cand.batch, m)),
                       timestamps=cand.timestamps[sel])
        y_c, _ = ops.hstu_layer_fwd_mfalcon(dims, wts, hist, uvqk_h, dev.jagged_of(mc),
                                            dev.bf16_tensor(xc[sel]))
        torch.cuda.synchronize()
        outs[sel] = dev.bf16_to_numpy(y_c)
    return dev.bf16_to_numpy(y_h), outs


def test_mfalcon_matches_oracle_and_microbatch_bitwise():
    w = wl.config(4, batch=4, seq_len=512)  # 4 users x (512 history + 128 candidates)
    d = w.dims
    say(f"[mfalcon] B={w.seq.batch} hist={w.seq.lengths[0]} cand={w.cand.lengths[0]}")
    y_h, y_c = _mfalcon(w, w.cand, w.x_cand, bm=128)
    _, y_c16 = _mfalcon(w, w.cand, w.x_cand, bm=16)
    assert np.array_equal(y_c.view(np.uint32), y_c16.view(np.uint32)), "b_m changed the result"
    want_h, want_c = ref.mfalcon_fwd(w.x, w.seq.offsets, w.seq.timestamps, w.x_cand, w.cand.offsets,
                                     w.cand.timestamps, w.weights, d.num_heads, d.dqk, d.dv, d.ln_eps)
    for name, got, want in (("history", y_h, want_h), ("candidates", y_c, want_c)):
        err = np.abs(got.astype(np.float64) - want)
        say(f"        {name}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}")
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS


@pytest.mark.parametrize("lengths,cap_extra,d_model,heads,dh", [
    ([37, 0, 91, 5], 163, 128, 2, 64),       # the 128-tile GEMM path (M < 256)
    ([300, 1, 512, 77], 700, 256, 4, 64),    # the 256-tile GEMM path, ragged tails
])
def test_token_capacity_matches_exact_count(lengths, cap_extra, d_model, heads, dh):
    """total_tokens above seq_offsets[B] (a capacity): the layer, the training forward, a
    2-layer stack and the attention alone give the exact-count results bit for bit, and
    rows from seq_offsets[B] on are left as they were."""
    d = wl.LayerDims(d_model=d_model, num_heads=heads, dqk=dh, dv=dh)
    w = wl.random_layer(77, lengths, d)
    T = w.seq.total
    cap = T + cap_extra
    dims, wts = dev.dims_of(d), dev.weights_of(w.weights)
    exact = dev.jagged_of(w.seq)
    capj = dev.jagged_of(w.seq)
    capj.total_tokens = cap
    ts = torch.zeros(cap, dtype=torch.int32, device="cuda")
    ts[:T] = capj.timestamps
    capj.timestamps = ts
    xc = torch.zeros((cap, d.d_model), dtype=torch.bfloat16, device="cuda")
    xc[:T] = dev.bf16_tensor(w.x)
    say(f"[capacity] lengths {lengths} T={T} capacity={cap} d={d_model} {heads}x{dh}")
    y0, u0 = ops.hstu_layer_fwd(dims, wts, exact, xc[:T])
    y1 = torch.full((cap, d.d_model), 7.0, dtype=torch.bfloat16, device="cuda")
    u1 = torch.full((cap, d.uvqk_width), 7.0, dtype=torch.float16, device="cuda")
    ops.hstu_layer_fwd(dims, wts, capj, xc, y=y1, uvqk=u1)
    lw = [wts, dev.weights_of(wl.draw_weights(np.random.default_rng(78), d))]
    s0, _ = ops.hstu_stack_fwd(dims, lw, exact, xc[:T])
    s1 = torch.full((cap, d.d_model), 7.0, dtype=torch.bfloat16, device="cuda")
    ops.hstu_stack_fwd(dims, lw, capj, xc, y=s1)
    hq = heads * dh
    q, k, v = u0[:, 2 * hq:3 * hq], u0[:, 3 * hq:], u0[:, hq:2 * hq]
    a0 = ops.hstu_attn_fwd(dims, exact, q, k, v, row_stride=u0.stride(0),
                           rab_pos=wts.rab_pos, rab_time=wts.rab_time)
    ucap = torch.zeros((cap, d.uvqk_width), dtype=torch.float16, device="cuda")
    ucap[:T] = u0
    qc, kc, vc = ucap[:, 2 * hq:3 * hq], ucap[:, 3 * hq:], ucap[:, hq:2 * hq]
    a1 = torch.full((cap, hq), 7.0, dtype=torch.float32, device="cuda")
    ops.hstu_attn_fwd(dims, capj, qc, kc, vc, row_stride=ucap.stride(0), rab_pos=wts.rab_pos,
                      rab_time=wts.rab_time, out=a1)
    torch.cuda.synchronize()
    assert torch.equal(y1[:T].view(torch.int16), y0.view(torch.int16))
    assert torch.equal(u1[:T].view(torch.int16), u0.view(torch.int16))
    assert torch.all(y1[T:] == 7.0) and torch.all(u1[T:] == 7.0)
    assert torch.equal(s1[:T].view(torch.int16), s0.view(torch.int16))
    assert torch.all(s1[T:] == 7.0)
    assert torch.equal(a1[:T], a0) and torch.all(a1[T:] == 7.0)
    # the training forward: y, U|V|Q|K and the attention output's parts
    t0 = ops.hstu_layer_fwd_train(dims, wts, exact, xc[:T])
    t1 = (torch.full((cap, d.d_model), 7.0, dtype=torch.bfloat16, device="cuda"),
          torch.full((cap, d.uvqk_width), 7.0, dtype=torch.float16, device="cuda"),
          torch.full((cap, heads * dh), 7.0, dtype=torch.float16, device="cuda"),
          torch.full((cap, heads, 2), 7.0, dtype=torch.float32, device="cuda"))
    ops.hstu_layer_fwd_train(dims, wts, capj, xc, y=t1[0], uvqk=t1[1], cn=t1[2], stats=t1[3])
    torch.cuda.synchronize()
    assert torch.equal(t0[0].view(torch.int16), y0.view(torch.int16))
    for a, b in zip(t0, t1):
        assert torch.equal(b[:T], a) and torch.all(b[T:] == 7.0)
