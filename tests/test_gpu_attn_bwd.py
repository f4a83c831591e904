"""GPU parity of the attention gradients (hstu_attn_bwd) against the fp64 oracle.

dQ, dK and dV from the HIP kernels are compared element by element with
oracle/hstu_bwd.attention_bwd on the same fp16-exact Q, K, V and the same fp32 upstream
gradient, on jagged batches with empty, one-token and ragged users, at head sizes 32, 64
and 128, with shared and per-head bias tables.  Bar: the error divided by the standard
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


def _case(seed, lengths, H, dh, per_head, scale=0.25):
    rng = np.random.default_rng(seed)
    seq = wl.jagged_from_lengths(rng, lengths)
    T = seq.total
    q, k, v = (wl.round_f16(scale * rng.standard_normal((T, H * dh), dtype=np.float32))
               for _ in range(3))
    P = (0.5 * rng.standard_normal((H if per_head else 1, 64))).astype(np.float32)
    Tt = (0.5 * rng.standard_normal((H if per_head else 1, 32))).astype(np.float32)
    g = rng.standard_normal((T, H * dh)).astype(np.float32)
    return seq, q, k, v, P, Tt, g


def _gpu_bwd(seq, q, k, v, P, Tt, g, H, dh):
    dims = ops.LayerDims(d_model=max(64, H * dh), num_heads=H, dqk=dh, dv=dh, pos_buckets=64,
                         time_buckets=32, rab_heads=P.shape[0])
    buf = dev.f16_tensor(np.concatenate([q, k, v], axis=1))
    hq = H * dh
    return ops.hstu_attn_bwd(dims, dev.jagged_of(seq), buf[:, :hq], buf[:, hq:2 * hq],
                             buf[:, 2 * hq:], torch.from_numpy(g).cuda(), row_stride=buf.stride(0),
                             rab_pos=torch.from_numpy(P).cuda(), rab_time=torch.from_numpy(Tt).cuda())


@pytest.mark.parametrize("seed,lengths,H,dh,per_head", [
    (0, [5, 17, 32, 64, 0, 1, 100], 2, 32, False),
    (1, [33, 200, 7, 129], 2, 64, True),
    (2, [300, 45, 0, 160], 2, 128, False),
])
def test_attention_gradients_match_oracle(seed, lengths, H, dh, per_head):
    seq, q, k, v, P, Tt, g = _case(seed, lengths, H, dh, per_head)
    say(f"[bwd] lengths={lengths} H={H} dh={dh} per_head_rab={per_head}")
    got = _gpu_bwd(seq, q, k, v, P, Tt, g, H, dh)
    torch.cuda.synchronize()
    again = _gpu_bwd(seq, q, k, v, P, Tt, g, H, dh)
    torch.cuda.synchronize()
    want = bwd.attention_bwd(q, k, v, g, seq.offsets, seq.timestamps, H, dh, dh, P, Tt)
    for name, gt, ag, wt in zip(("dq", "dk", "dv"), got, again, want[:3]):
        gn = gt.cpu().numpy().astype(np.float64)
        assert np.array_equal(gt.cpu().numpy(), ag.cpu().numpy()), f"{name} not deterministic"
        sd = float(np.std(wt)) or 1.0
        err = np.abs(gn - wt) / sd
        say(f"      {name}: max_rel={err.max():.3e} mean_rel={err.mean():.3e} (std {sd:.3g})")
        assert np.all(np.isfinite(gn))
        assert err.max() <= MAX_REL and err.mean() <= MEAN_REL, name
