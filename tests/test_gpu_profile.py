"""GPU checks of the library's optional event timing: a kernel selection times only the
selected launches, and the shader clock read inside the profiled attention launches is a
plausible frequency (and reads 0 after a reset)."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from hstu_pointwise_attention_jagged_amd import device as dev  # noqa: E402
from hstu_pointwise_attention_jagged_amd import ops  # noqa: E402
from hstu_pointwise_attention_jagged_amd import workloads as wl  # noqa: E402

pytestmark = pytest.mark.gpu


def test_selected_kernel_timing_and_clock():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    w = wl.config(1)
    d = w.dims
    dims, seq = dev.dims_of(d), dev.jagged_of(w.seq)
    wts = dev.weights_of(w.weights)
    x = dev.bf16_tensor(w.x)
    ops.hstu_layer_fwd(dims, wts, seq, x)  # warm
    torch.cuda.synchronize()
    print("[profile] layer of the 64-user batch, attention only", flush=True)
    ops.profile_reset()
    ops.profile_enable(True, kernels=["attention"])
    ops.hstu_layer_fwd(dims, wts, seq, x)
    ops.hstu_layer_fwd(dims, wts, seq, x)
    torch.cuda.synchronize()
    ops.profile_enable(False)
    k = ops.profile_collect()
    assert k["attention"][1] == 2 and k["attention"][0] > 0.0
    assert all(v[1] == 0 for name, v in k.items() if name != "attention"), k
    ghz = ops.profile_clock_ghz()
    print(f"      clock {ghz:.3f} GHz", flush=True)
    assert 0.3 < ghz < 3.5
    ops.profile_reset()
    assert ops.profile_clock_ghz() == 0.0
    # every kernel
    ops.profile_enable(True)
    ops.hstu_layer_fwd(dims, wts, seq, x)
    torch.cuda.synchronize()
    ops.profile_enable(False)
    k = ops.profile_collect()
    ops.profile_reset()
    assert all(k[name][1] >= 1 for name in ("schedule", "f1_gemm_silu", "attention", "f2_gemm"))
    assert k["f2_prep"][1] == 0  # the w2 conversion is part of the f1 launch (id 1)
