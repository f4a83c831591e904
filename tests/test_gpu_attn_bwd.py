"""GPU parity of the attention gradients (hstu_attn_bwd) against the fp64 oracle.

dQ, dK and dV from the HIP kernels are compared element by element with
oracle/hstu_bwd.attention_bwd on the same fp16-exact Q, K, V and the same fp32 upstream
gradient, on jagged batches with empty, one-token and ragged users, at head sizes 32, 64
and 128, with shared and per-head bias tables (whose gradients are compared too), and at the
full 8 x 8192-token size (8 heads
of 128, the launch that bench.py times) on sampled rows that the oracle computes one by
one: first and last rows of sequences, both sides of a 128-row tile edge, and the middle
of a sequence.  Bar: the error divided by the standard
deviation of the oracle's tensor, max <= 2e-2 and mean <= 2e-3 (the bar of the raw
attention output; the kernels round dO, A and dS to fp16 for the matrix products).  Two
runs must agree bit for bit.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from hstu_pointwise_attention_jagged_amd import device as dev  # noqa: E402
from hstu_pointwise_attention_jagged_amd import ops  # noqa: E402
from hstu_pointwise_attention_jagged_amd import workloads as wl  # noqa: E402
from oracle import hstu_bwd as bwd  # noqa: E402

pytestmark = pytest.mark.gpu

MAX_REL, MEAN_REL = 2e-2, 2e-3


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _case(seed, lengths, H, dh, per_head, scale=0.25, g_scale=1.0, pos_buckets=64,
          time_buckets=32):
    rng = np.random.default_rng(seed)
    seq = wl.jagged_from_lengths(rng, lengths)
    T = seq.total
    q, k, v = (wl.round_f16(scale * rng.standard_normal((T, H * dh), dtype=np.float32))
               for _ in range(3))
    P = (0.5 * rng.standard_normal((H if per_head else 1, pos_buckets))).astype(np.float32)
    Tt = (0.5 * rng.standard_normal((H if per_head else 1, time_buckets))).astype(np.float32)
    g = (g_scale * rng.standard_normal((T, H * dh))).astype(np.float32)
    return seq, q, k, v, P, Tt, g


def _gpu_bwd(seq, q, k, v, P, Tt, g, H, dh, path="stored"):
    rows = (P if P is not None else Tt if Tt is not None else np.zeros((1, 1))).shape[0]
    dims = ops.LayerDims(d_model=max(64, H * dh), num_heads=H, dqk=dh, dv=dh,
                         pos_buckets=P.shape[1] if P is not None else 64,
                         time_buckets=Tt.shape[1] if Tt is not None else 32, rab_heads=rows)
    buf = dev.f16_tensor(np.concatenate([q, k, v], axis=1))
    hq = H * dh
    opt = lambda a: None if a is None else torch.from_numpy(a).cuda()  # noqa: E731
    js = dev.jagged_of(seq)
    # "stored": the workspace that keeps dS for the dQ kernel; "recompute": the minimum,
    # with which the dQ kernel forms dS again
    ws = torch.empty(max(256, ops.hstu_attn_bwd_workspace_bytes(dims, js, minimum=path == "recompute")),
                     dtype=torch.uint8, device="cuda")
    return ops.hstu_attn_bwd(dims, js, buf[:, :hq], buf[:, hq:2 * hq], buf[:, 2 * hq:],
                             torch.from_numpy(g).cuda(), row_stride=buf.stride(0), rab_pos=opt(P),
                             rab_time=opt(Tt), rab_grads=True, workspace=ws)


# (seed, lengths, H, dh, per-head tables, dO scale, position buckets, time buckets, tables)
CASES = [
    (0, [5, 17, 32, 64, 0, 1, 100], 2, 32, False, 1.0, 64, 32, True),
    (1, [33, 200, 7, 129], 2, 64, True, 1.0, 64, 32, True),
    (2, [300, 45, 0, 160], 2, 128, False, 1.0, 64, 32, True),
    # long rows, few position buckets: most blocks take one or two bias values
    (3, [1500, 700, 31], 1, 64, False, 1e-7, 8, 16, True),     # tiny upstream gradient
    (4, [1000, 97], 2, 128, True, 300.0, 8, 16, True),         # large upstream gradient
    (5, [400, 129], 2, 128, False, 1.0, 64, 32, False),        # no bias tables
]


@pytest.mark.parametrize("path", ["stored", "recompute"])
@pytest.mark.parametrize("seed,lengths,H,dh,per_head,g_scale,pb,tb,tables", CASES)
def test_attention_gradients_match_oracle(seed, lengths, H, dh, per_head, g_scale, pb, tb, tables,
                                          path):
    seq, q, k, v, P, Tt, g = _case(seed, lengths, H, dh, per_head, g_scale=g_scale,
                                   pos_buckets=pb, time_buckets=tb)
    if not tables:
        P = Tt = None
    say(f"[bwd] {path} lengths={lengths} H={H} dh={dh} per_head_rab={per_head} dO x{g_scale} "
        f"buckets={pb}/{tb} tables={tables}")
    got = _gpu_bwd(seq, q, k, v, P, Tt, g, H, dh, path)
    torch.cuda.synchronize()
    again = _gpu_bwd(seq, q, k, v, P, Tt, g, H, dh, path)
    torch.cuda.synchronize()
    want = bwd.attention_bwd(q, k, v, g, seq.offsets, seq.timestamps, H, dh, dh, P, Tt)
    for name, gt, ag, wt in zip(("dq", "dk", "dv", "d_rab_pos", "d_rab_time"), got, again, want):
        if wt is None:
            assert gt is None
            continue
        gn = gt.cpu().numpy().astype(np.float64)
        if name.startswith("d_rab"):
            # LDS atomics order a wave's lanes as the hardware does: equal to rounding only
            a, b = gt.cpu().numpy().astype(np.float64), ag.cpu().numpy().astype(np.float64)
            assert np.abs(a - b).max() <= 1e-5 * max(np.abs(a).max(), 1e-30), f"{name} not repeatable"
        else:
            assert np.array_equal(gt.cpu().numpy(), ag.cpu().numpy()), f"{name} not deterministic"
        sd = float(np.std(wt)) or 1.0
        err = np.abs(gn - wt) / sd
        say(f"      {name}: max_rel={err.max():.3e} mean_rel={err.mean():.3e} (std {sd:.3g})")
        assert np.all(np.isfinite(gn))
        assert err.max() <= MAX_REL and err.mean() <= MEAN_REL, name


def test_upstream_gradient_maximum_off_every_fourth_column():
    """The scale of the fp16 copy of dO comes from max |dO| over every element.  An upstream
    gradient that is zero except large entries in columns 1, 2 and 3 (mod 4) must be scaled
    by its true maximum: otherwise the entries overflow fp16 and the gradients turn
    non-finite."""
    H, dh = 2, 64
    seq, q, k, v, P, Tt, _ = _case(21, [40, 130, 7], H, dh, False)
    g = np.zeros((seq.total, H * dh), np.float32)
    rng = np.random.default_rng(22)
    rows = rng.integers(0, seq.total, 12)
    cols = 4 * rng.integers(0, H * dh // 4, 12) + 1 + np.arange(12) % 3
    g[rows, cols] = 1e6 * (1.0 + rng.random(12)).astype(np.float32)
    say("[bwd] dO with its maximum off the columns 0 mod 4")
    got = _gpu_bwd(seq, q, k, v, P, Tt, g, H, dh)
    torch.cuda.synchronize()
    want = bwd.attention_bwd(q, k, v, g, seq.offsets, seq.timestamps, H, dh, dh, P, Tt)
    for name, gt, wt in zip(("dq", "dk", "dv"), got, want):
        gn = gt.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(gn)), name
        err = np.abs(gn - wt) / float(np.std(wt))
        say(f"      {name}: max_rel={err.max():.3e} mean_rel={err.mean():.3e}")
        assert err.max() <= MAX_REL and err.mean() <= MEAN_REL, name


def test_zero_upstream_gradient_gives_zero():
    seq, q, k, v, P, Tt, g = _case(6, [70, 130], 2, 64, False)
    g[:] = 0.0
    say("[bwd] dO = 0")
    for t in _gpu_bwd(seq, q, k, v, P, Tt, g, 2, 64):
        assert t is None or torch.count_nonzero(t).item() == 0


def test_attention_gradients_full_size_sampled_rows():
    w = wl.config(2)
    d = w.dims
    H, dh = d.num_heads, d.dqk
    seq = w.seq
    rng = np.random.default_rng(2002)
    q, k, v, g = wl.draw_attention_grad_inputs(rng, seq.total, H * dh)
    P, Tt = w.weights.rab_pos, w.weights.rab_time
    say(f"[bwd full] B={seq.batch} T={seq.total} H={H} dh={dh}")
    got = _gpu_bwd(seq, q, k, v, P, Tt, g, H, dh)
    torch.cuda.synchronize()
    off = seq.offsets.astype(np.int64)
    rows = [0, 1, 127, 128, 4095, 8191, int(off[3]) + 2000, int(off[7]) + 8063,
            int(off[7]) + 8064, int(off[8]) - 1]
    want = bwd.attention_bwd(q, k, v, g, off, seq.timestamps, H, dh, dh, P, Tt, rows=rows)
    for name, gt, wt in zip(("dq", "dk", "dv"), got[:3], want[:3]):
        gn = gt[rows].cpu().numpy().astype(np.float64)
        wr = wt[rows]
        sd = float(np.std(wr)) or 1.0
        err = np.abs(gn - wr) / sd
        say(f"      {name}: max_rel={err.max():.3e} mean_rel={err.mean():.3e} (std {sd:.3g})")
        assert np.all(np.isfinite(gn))
        assert err.max() <= MAX_REL and err.mean() <= MEAN_REL, name
