"""Copies seeded workloads (NumPy) onto the GPU as the tensors the binding expects.

Transfers only: bf16 bit patterns are reinterpreted, fp32/int32 arrays are copied as is.
"""

from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import workloads as wl
from .ops import DeviceJagged, DeviceWeights, LayerDims


def bf16_tensor(x_f32: np.ndarray, device="cuda") -> torch.Tensor:
    """bf16 device tensor holding the bf16-exact fp32 array ``x_f32``."""
    bits = wl.bf16_bits(x_f32)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)


def f16_tensor(x: np.ndarray, device="cuda") -> torch.Tensor:
    """fp16 device tensor of the fp16-exact array ``x``."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float16)).to(device)


def f32_tensor(a: Optional[np.ndarray], device="cuda") -> Optional[torch.Tensor]:
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def i32_tensor(a: Optional[np.ndarray], device="cuda") -> Optional[torch.Tensor]:
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def dims_of(d: wl.LayerDims) -> LayerDims:
    return LayerDims(d.d_model, d.num_heads, d.dqk, d.dv, d.pos_buckets, d.time_buckets,
                     d.rab_heads, d.ln_eps)


def weights_of(w: wl.LayerWeights, device="cuda") -> DeviceWeights:
    return DeviceWeights(w1=bf16_tensor(w.w1, device), w2=bf16_tensor(w.w2, device),
                         b1=f32_tensor(w.b1, device), b2=f32_tensor(w.b2, device),
                         ln_gamma=f32_tensor(w.ln_gamma, device), ln_beta=f32_tensor(w.ln_beta, device),
                         rab_pos=f32_tensor(w.rab_pos, device), rab_time=f32_tensor(w.rab_time, device))


def jagged_of(s: wl.Jagged, device="cuda", with_time: bool = True) -> DeviceJagged:
    lengths = s.lengths
    return DeviceJagged(offsets=i32_tensor(s.offsets, device), total_tokens=s.total,
                        max_seq_len=int(lengths.max()) if lengths.size else 0,
                        timestamps=i32_tensor(s.timestamps, device) if with_time else None)


def bf16_to_numpy(t: torch.Tensor) -> np.ndarray:
    """Exact fp32 values of a bf16 device tensor."""
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return wl.bf16_to_f32(bits)
