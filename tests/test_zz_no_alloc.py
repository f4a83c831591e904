"""hstu_attn_fwd_noalloc (the attention forward whose scratch is the library's static
per-GPU array) against hstu_attn_fwd with a caller workspace: the same kernels, so the
outputs must agree bit for bit, over consecutive calls whose sizes shrink (the array
keeps the previous call's contents)."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from hstu_pointwise_attention_jagged_amd import device as dev  # noqa: E402
from hstu_pointwise_attention_jagged_amd import ops  # noqa: E402
from hstu_pointwise_attention_jagged_amd import workloads as wl  # noqa: E402

pytestmark = pytest.mark.gpu


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


def _case(seed, lengths, H, dh, prefix_lengths=None):
    rng = np.random.default_rng(seed)
    seq = wl.jagged_from_lengths(rng, lengths)
    T = seq.total
    qkv = wl.round_f16(rng.standard_normal((T, 3 * H * dh), dtype=np.float32))
    P = (0.5 * rng.standard_normal((1, 64))).astype(np.float32)
    Tt = (0.5 * rng.standard_normal((1, 32))).astype(np.float32)
    dims = ops.LayerDims(d_model=max(64, H * dh), num_heads=H, dqk=dh, dv=dh)
    buf = dev.f16_tensor(qkv)
    hq = H * dh
    args = dict(row_stride=buf.stride(0), rab_pos=dev.f32_tensor(P), rab_time=dev.f32_tensor(Tt))
    pref, mask = None, "causal"
    if prefix_lengths is not None:
        hist = wl.jagged_from_lengths(rng, prefix_lengths)
        pbuf = dev.f16_tensor(wl.round_f16(rng.standard_normal((hist.total, 3 * hq), dtype=np.float32)))
        last = np.array([hist.timestamps[hist.offsets[b + 1] - 1] if prefix_lengths[b] else 0
                         for b in range(len(lengths))])
        seq.timestamps = np.repeat(last + 7, lengths).astype(np.int32)
        pref = (dev.jagged_of(hist), pbuf[:, :hq], pbuf[:, hq:2 * hq], pbuf.stride(0))
        mask = "self_only"
    return dims, dev.jagged_of(seq), buf[:, :hq], buf[:, hq:2 * hq], buf[:, 2 * hq:], args, pref, mask


@pytest.mark.parametrize("cases", [[
    (71, [300, 0, 1000, 17, 129], 2, 128, None),   # first call: the largest
    (72, [5, 64, 33], 4, 64, None),                # second call: smaller
    (73, [7, 1, 130, 3], 2, 64, [100, 0, 257, 64]),  # smaller still, candidates + prefix
]])
def test_noalloc_matches_workspace_entry_point(cases):
    assert ops.hstu_attn_noalloc_max_scratch_bytes() == 16 << 20
    for seed, lengths, H, dh, pl in cases:
        say(f"[noalloc] seed={seed} lengths={lengths} H={H} dh={dh} prefix={pl}")
        dims, seq, q, k, v, args, pref, mask = _case(seed, lengths, H, dh, pl)
        want = ops.hstu_attn_fwd(dims, seq, q, k, v, prefix=pref, mask=mask, **args)
        got = torch.full_like(want, float("nan"))
        ops.hstu_attn_fwd_noalloc(dims, seq, q, k, v, got, prefix=pref, mask=mask, **args)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), "outputs differ"
