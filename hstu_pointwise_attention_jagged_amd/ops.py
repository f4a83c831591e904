"""Python entry points over libhstu's C ABI (same names as the C functions).

PyTorch supplies device memory and the stream; these wrappers only check tensor
dtypes/devices, fill the ctypes structures, allocate outputs and workspace when the
caller does not pass them, and call the library.  Every step of the computation runs in
the HIP kernels behind ``include/hstu.h``.
"""

from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from . import _lib

__all__ = ["HSTUError", "LayerDims", "DeviceWeights", "DeviceJagged", "hstu_layer_fwd",
           "hstu_layer_fwd_mfalcon", "hstu_attn_fwd", "hstu_attn_fwd_noalloc", "hstu_attn_noalloc_max_scratch_bytes",
           "hstu_layer_workspace_bytes",
           "hstu_attn_workspace_bytes", "hstu_mfalcon_workspace_bytes", "hstu_validate_jagged",
           "hstu_sl_workspace_bytes", "hstu_stochastic_length", "hstu_stack_fwd",
           "hstu_stack_fwd_mfalcon", "hstu_stack_workspace_bytes",
           "hstu_stack_mfalcon_workspace_bytes", "hstu_attn_bwd", "hstu_attn_bwd_workspace_bytes",
           "hstu_layer_bwd", "hstu_layer_bwd_workspace_bytes",
           "profile_enable", "profile_reset", "profile_collect", "profile_clock_ghz"]


class HSTUError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _lib.load()
        msg = lib.hstu_status_str(status).decode()
        if status == _lib.HSTU_ERR_HIP:
            msg += f" (hip error {lib.hstu_last_hip_error()})"
        super().__init__(f"{where}: {msg}")
        self.status = status


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

    def c(self) -> _lib.Dims:
        return _lib.Dims(self.d_model, self.num_heads, self.dqk, self.dv, self.pos_buckets,
                         self.time_buckets, self.rab_heads, self.ln_eps)

    @property
    def uvqk_width(self) -> int:
        return 2 * self.num_heads * (self.dqk + self.dv)

    @property
    def hdv(self) -> int:
        return self.num_heads * self.dv


@dataclasses.dataclass
class DeviceWeights:
    w1: torch.Tensor                        # bf16 [2H(dv+dqk)][d]
    w2: torch.Tensor                        # bf16 [d][H*dv]
    b1: Optional[torch.Tensor] = None       # fp32
    b2: Optional[torch.Tensor] = None
    ln_gamma: Optional[torch.Tensor] = None
    ln_beta: Optional[torch.Tensor] = None
    rab_pos: Optional[torch.Tensor] = None  # fp32 [rab_heads][pos_buckets]
    rab_time: Optional[torch.Tensor] = None

    def c(self) -> _lib.Weights:
        _check(self.w1, torch.bfloat16, "w1")
        _check(self.w2, torch.bfloat16, "w2")
        for n in ("b1", "b2", "ln_gamma", "ln_beta", "rab_pos", "rab_time"):
            t = getattr(self, n)
            if t is not None:
                _check(t, torch.float32, n)
        return _lib.Weights(*(_ptr(getattr(self, n)) for n in
                              ("w1", "b1", "w2", "b2", "ln_gamma", "ln_beta", "rab_pos", "rab_time")))


@dataclasses.dataclass
class DeviceJagged:
    offsets: torch.Tensor                   # int32 [B+1] on the device
    total_tokens: int                       # host copy of offsets[B] (forward calls: or a capacity above it)
    max_seq_len: int                        # host upper bound on lengths
    timestamps: Optional[torch.Tensor] = None  # int32 [T] on the device

    @property
    def batch(self) -> int:
        return int(self.offsets.shape[0]) - 1

    def c(self) -> _lib.Jagged:
        _check(self.offsets, torch.int32, "seq_offsets")
        if self.timestamps is not None:
            _check(self.timestamps, torch.int32, "timestamps")
        return _lib.Jagged(self.batch, int(self.total_tokens), int(self.max_seq_len),
                           _ptr(self.offsets), _ptr(self.timestamps))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _check(t: torch.Tensor, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _raise(status: int, where: str):
    if status != _lib.HSTU_OK:
        raise HSTUError(status, where)


def hstu_layer_workspace_bytes(dims: LayerDims, seq: DeviceJagged) -> int:
    lib = _lib.load()
    d, s = dims.c(), seq.c()
    return int(lib.hstu_layer_workspace_bytes(ctypes.byref(d), ctypes.byref(s)))


def hstu_attn_workspace_bytes(dims: LayerDims, seq: DeviceJagged,
                              prefix_seq: Optional[DeviceJagged] = None) -> int:
    lib = _lib.load()
    d, s = dims.c(), seq.c()
    ps = prefix_seq.c() if prefix_seq is not None else None
    return int(lib.hstu_attn_workspace_bytes(ctypes.byref(d), ctypes.byref(s),
                                             ctypes.byref(ps) if ps is not None else None))


def hstu_mfalcon_workspace_bytes(dims: LayerDims, hist: DeviceJagged, cand: DeviceJagged) -> int:
    lib = _lib.load()
    d, h, c = dims.c(), hist.c(), cand.c()
    return int(lib.hstu_mfalcon_workspace_bytes(ctypes.byref(d), ctypes.byref(h), ctypes.byref(c)))


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    if ws is not None:
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def hstu_layer_fwd(dims: LayerDims, w: DeviceWeights, seq: DeviceJagged, x: torch.Tensor, *,
                   y: Optional[torch.Tensor] = None, uvqk: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None):
    """One HSTU layer (causal).  Returns (y bf16 [T][d], uvqk fp16 [T][2H(dv+dqk)])."""
    lib = _lib.load()
    _check(x, torch.bfloat16, "x")
    T = seq.total_tokens
    if y is None:
        y = torch.empty((T, dims.d_model), dtype=torch.bfloat16, device=x.device)
    if uvqk is None:
        uvqk = torch.empty((T, dims.uvqk_width), dtype=torch.float16, device=x.device)
    _check(y, torch.bfloat16, "y")
    _check(uvqk, torch.float16, "uvqk")
    d, wc, s = dims.c(), w.c(), seq.c()
    need = int(lib.hstu_layer_workspace_bytes(ctypes.byref(d), ctypes.byref(s)))
    ws = _workspace(need, x.device, workspace)
    st = lib.hstu_layer_fwd(ctypes.byref(d), ctypes.byref(wc), ctypes.byref(s), _ptr(x), _ptr(y),
                            _ptr(uvqk), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _raise(st, "hstu_layer_fwd")
    return y, uvqk


def hstu_layer_fwd_train(dims: LayerDims, w: DeviceWeights, seq: DeviceJagged, x: torch.Tensor, *,
                         y: Optional[torch.Tensor] = None, uvqk: Optional[torch.Tensor] = None,
                         cn: Optional[torch.Tensor] = None, stats: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None):
    """hstu_layer_fwd that also returns what hstu_layer_bwd_saved reuses.  Returns
    (y bf16 [T][d], uvqk fp16 [T][2H(dv+dqk)], cn fp16 [T][H*dv], stats fp32 [T][H][2])."""
    lib = _lib.load()
    _check(x, torch.bfloat16, "x")
    T = seq.total_tokens
    if y is None:
        y = torch.empty((T, dims.d_model), dtype=torch.bfloat16, device=x.device)
    if uvqk is None:
        uvqk = torch.empty((T, dims.uvqk_width), dtype=torch.float16, device=x.device)
    if cn is None:
        cn = torch.empty((T, dims.hdv), dtype=torch.float16, device=x.device)
    if stats is None:
        stats = torch.empty((T, dims.num_heads, 2), dtype=torch.float32, device=x.device)
    _check(y, torch.bfloat16, "y")
    _check(uvqk, torch.float16, "uvqk")
    _check(cn, torch.float16, "cn")
    _check(stats, torch.float32, "stats")
    d, wc, s = dims.c(), w.c(), seq.c()
    need = int(lib.hstu_layer_workspace_bytes(ctypes.byref(d), ctypes.byref(s)))
    ws = _workspace(need, x.device, workspace)
    st = lib.hstu_layer_fwd_train(ctypes.byref(d), ctypes.byref(wc), ctypes.byref(s), _ptr(x), _ptr(y),
                                  _ptr(uvqk), _ptr(cn), _ptr(stats), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream))
    _raise(st, "hstu_layer_fwd_train")
    return y, uvqk, cn, stats


def hstu_layer_fwd_mfalcon(dims: LayerDims, w: DeviceWeights, hist: DeviceJagged,
                           hist_uvqk: torch.Tensor, cand: DeviceJagged, x_cand: torch.Tensor, *,
                           y_cand: Optional[torch.Tensor] = None,
                           uvqk_cand: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None):
    """M-FALCON candidate micro-batch against a cached history.  Returns (y_cand, uvqk_cand)."""
    lib = _lib.load()
    _check(x_cand, torch.bfloat16, "x_cand")
    _check(hist_uvqk, torch.float16, "hist_uvqk")
    T = cand.total_tokens
    if y_cand is None:
        y_cand = torch.empty((T, dims.d_model), dtype=torch.bfloat16, device=x_cand.device)
    if uvqk_cand is None:
        uvqk_cand = torch.empty((T, dims.uvqk_width), dtype=torch.float16, device=x_cand.device)
    _check(y_cand, torch.bfloat16, "y_cand")
    _check(uvqk_cand, torch.float16, "uvqk_cand")
    d, wc, hs, cs = dims.c(), w.c(), hist.c(), cand.c()
    need = int(lib.hstu_mfalcon_workspace_bytes(ctypes.byref(d), ctypes.byref(hs), ctypes.byref(cs)))
    ws = _workspace(need, x_cand.device, workspace)
    st = lib.hstu_layer_fwd_mfalcon(ctypes.byref(d), ctypes.byref(wc), ctypes.byref(hs),
                                    _ptr(hist_uvqk), ctypes.byref(cs), _ptr(x_cand), _ptr(y_cand),
                                    _ptr(uvqk_cand), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream))
    _raise(st, "hstu_layer_fwd_mfalcon")
    return y_cand, uvqk_cand


def _weights_array(ws):
    arr = (_lib.Weights * len(ws))()
    for i, w in enumerate(ws):
        arr[i] = w.c()
    return arr


def hstu_stack_workspace_bytes(dims: LayerDims, seq: DeviceJagged) -> int:
    lib = _lib.load()
    d, s = dims.c(), seq.c()
    return int(lib.hstu_stack_workspace_bytes(ctypes.byref(d), ctypes.byref(s)))


def hstu_stack_mfalcon_workspace_bytes(dims: LayerDims, hist: DeviceJagged, cand: DeviceJagged) -> int:
    lib = _lib.load()
    d, hs, cs = dims.c(), hist.c(), cand.c()
    return int(lib.hstu_stack_mfalcon_workspace_bytes(ctypes.byref(d), ctypes.byref(hs), ctypes.byref(cs)))


def hstu_stack_fwd(dims: LayerDims, weights, seq: DeviceJagged, x: torch.Tensor, *,
                   keep_caches: bool = False, y: Optional[torch.Tensor] = None,
                   uvqk: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   stream=None):
    """A stack of len(weights) causal layers.  Returns (y bf16 [T][d], uvqk): uvqk is
    [T][2H(dv+dqk)] scratch, or [L][T][2H(dv+dqk)] per-layer caches with keep_caches."""
    lib = _lib.load()
    _check(x, torch.bfloat16, "x")
    L, T = len(weights), seq.total_tokens
    if y is None:
        y = torch.empty((T, dims.d_model), dtype=torch.bfloat16, device=x.device)
    if uvqk is None:
        shape = (L, T, dims.uvqk_width) if keep_caches else (T, dims.uvqk_width)
        uvqk = torch.empty(shape, dtype=torch.float16, device=x.device)
    _check(y, torch.bfloat16, "y")
    _check(uvqk, torch.float16, "uvqk")
    arr = _weights_array(weights)
    d, s = dims.c(), seq.c()
    need = int(lib.hstu_stack_workspace_bytes(ctypes.byref(d), ctypes.byref(s)))
    ws = _workspace(need, x.device, workspace)
    st = lib.hstu_stack_fwd(ctypes.byref(d), L, arr, ctypes.byref(s), _ptr(x), _ptr(y), _ptr(uvqk),
                            1 if keep_caches else 0, _ptr(ws), ws.numel() * ws.element_size(),
                            _stream(stream))
    _raise(st, "hstu_stack_fwd")
    return y, uvqk


def hstu_stack_fwd_mfalcon(dims: LayerDims, weights, hist: DeviceJagged, hist_uvqk: torch.Tensor,
                           cand: DeviceJagged, x_cand: torch.Tensor, *,
                           y_cand: Optional[torch.Tensor] = None,
                           uvqk_cand: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None):
    """Candidates through len(weights) layers against per-layer history caches
    hist_uvqk [L][T_hist][2H(dv+dqk)].  Returns y_cand bf16 [T_cand][d]."""
    lib = _lib.load()
    _check(x_cand, torch.bfloat16, "x_cand")
    _check(hist_uvqk, torch.float16, "hist_uvqk")
    L, T = len(weights), cand.total_tokens
    if hist_uvqk.dim() != 3 or hist_uvqk.shape[0] != L:
        raise ValueError("hist_uvqk: expected [L][T_hist][2H(dv+dqk)] per-layer caches")
    if y_cand is None:
        y_cand = torch.empty((T, dims.d_model), dtype=torch.bfloat16, device=x_cand.device)
    if uvqk_cand is None:
        uvqk_cand = torch.empty((T, dims.uvqk_width), dtype=torch.float16, device=x_cand.device)
    _check(y_cand, torch.bfloat16, "y_cand")
    _check(uvqk_cand, torch.float16, "uvqk_cand")
    arr = _weights_array(weights)
    d, hs, cs = dims.c(), hist.c(), cand.c()
    need = int(lib.hstu_stack_mfalcon_workspace_bytes(ctypes.byref(d), ctypes.byref(hs),
                                                      ctypes.byref(cs)))
    ws = _workspace(need, x_cand.device, workspace)
    st = lib.hstu_stack_fwd_mfalcon(ctypes.byref(d), L, arr, ctypes.byref(hs), _ptr(hist_uvqk),
                                    ctypes.byref(cs), _ptr(x_cand), _ptr(y_cand), _ptr(uvqk_cand),
                                    _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _raise(st, "hstu_stack_fwd_mfalcon")
    return y_cand


def hstu_attn_fwd(dims: LayerDims, seq: DeviceJagged, q: torch.Tensor, k: torch.Tensor,
                  v: torch.Tensor, *, row_stride: Optional[int] = None,
                  rab_pos: Optional[torch.Tensor] = None, rab_time: Optional[torch.Tensor] = None,
                  prefix: Optional[tuple] = None, mask: str = "causal",
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Equation 2 alone, fp32 output [T][H*dv].

    q, k, v: fp16 views whose rows are ``row_stride`` elements apart (they may be column
    slices of one buffer).  prefix: (DeviceJagged, k_p, v_p, p_row_stride) or None, k_p
    and v_p fp16 as well.
    """
    lib = _lib.load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.float16 or not t.is_cuda:
            raise TypeError(f"{n}: expected an fp16 device tensor")
    if row_stride is None:
        row_stride = q.stride(0)
    T = seq.total_tokens
    if out is None:
        out = torch.empty((T, dims.hdv), dtype=torch.float32, device=q.device)
    _check(out, torch.float32, "out")
    d, s = dims.c(), seq.c()
    pref = None
    ps = None
    if prefix is not None:
        pseq, kp, vp, pstride = prefix
        for n, t in (("k_p", kp), ("v_p", vp)):
            if t.dtype != torch.float16 or not t.is_cuda:
                raise TypeError(f"{n}: expected an fp16 device tensor")
        ps = pseq.c()
        pref = _lib.Prefix(ctypes.pointer(ps), _ptr(kp), _ptr(vp), int(pstride))
    need = int(lib.hstu_attn_workspace_bytes(ctypes.byref(d), ctypes.byref(s),
                                             ctypes.byref(ps) if ps is not None else None))
    ws = _workspace(need, q.device, workspace)
    m = {"causal": _lib.MASK_CAUSAL, "self_only": _lib.MASK_SELF_ONLY}[mask]
    st = lib.hstu_attn_fwd(ctypes.byref(d), _ptr(rab_pos), _ptr(rab_time), ctypes.byref(s),
                           _ptr(q), _ptr(k), _ptr(v), int(row_stride),
                           ctypes.byref(pref) if pref is not None else None, m, _ptr(out),
                           _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _raise(st, "hstu_attn_fwd")
    return out


def hstu_attn_noalloc_max_scratch_bytes() -> int:
    return int(_lib.load().hstu_attn_noalloc_max_scratch_bytes())


def hstu_attn_fwd_noalloc(dims: LayerDims, seq: DeviceJagged, q: torch.Tensor, k: torch.Tensor,
                          v: torch.Tensor, out: torch.Tensor, *, row_stride: Optional[int] = None,
                          rab_pos: Optional[torch.Tensor] = None,
                          rab_time: Optional[torch.Tensor] = None, prefix: Optional[tuple] = None,
                          mask: str = "causal", stream=None) -> torch.Tensor:
    """hstu_attn_fwd without a workspace (the library's static per-GPU scratch); the
    caller passes the fp32 output [T][H*dv].  Arguments as for hstu_attn_fwd."""
    lib = _lib.load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.float16 or not t.is_cuda:
            raise TypeError(f"{n}: expected an fp16 device tensor")
    _check(out, torch.float32, "out")
    if row_stride is None:
        row_stride = q.stride(0)
    d, s = dims.c(), seq.c()
    pref = None
    if prefix is not None:
        pseq, kp, vp, pstride = prefix
        for n, t in (("k_p", kp), ("v_p", vp)):
            if t.dtype != torch.float16 or not t.is_cuda:
                raise TypeError(f"{n}: expected an fp16 device tensor")
        ps = pseq.c()
        pref = _lib.Prefix(ctypes.pointer(ps), _ptr(kp), _ptr(vp), int(pstride))
    m = {"causal": _lib.MASK_CAUSAL, "self_only": _lib.MASK_SELF_ONLY}[mask]
    st = lib.hstu_attn_fwd_noalloc(ctypes.byref(d), _ptr(rab_pos), _ptr(rab_time), ctypes.byref(s),
                                   _ptr(q), _ptr(k), _ptr(v), int(row_stride),
                                   ctypes.byref(pref) if pref is not None else None, m, _ptr(out),
                                   _stream(stream))
    _raise(st, "hstu_attn_fwd_noalloc")
    return out


def hstu_sl_workspace_bytes(raw: DeviceJagged) -> int:
    lib = _lib.load()
    s = raw.c()
    return int(lib.hstu_sl_workspace_bytes(ctypes.byref(s)))


def hstu_stochastic_length(raw: DeviceJagged, u_keep: torch.Tensor, keys: torch.Tensor, *,
                           n_target: int = 4096, alpha: float = 1.6,
                           x: Optional[torch.Tensor] = None, gather_timestamps: bool = True,
                           workspace: Optional[torch.Tensor] = None, stream=None):
    """Stochastic Length over a raw batch (see include/hstu.h).

    u_keep: float64 [B] uniform draws; keys: int32 [T_raw] holding the 32-bit priorities'
    bit patterns (torch has no uint32 arithmetic dtype); x: optional 16-bit rows
    [T_raw][d] to gather.  Returns (kept int32 [T_raw], new_offsets int32 [B+1],
    new_ts int32 [T_raw] or None, x_out [T_raw][d] or None): the first new_offsets[B]
    entries of kept / new_ts / x_out are the new batch, the rest is left unwritten.
    """
    lib = _lib.load()
    _check(u_keep, torch.float64, "u_keep")
    _check(keys, torch.int32, "keys")
    dev = raw.offsets.device
    T = raw.total_tokens
    kept = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    new_off = torch.empty(raw.batch + 1, dtype=torch.int32, device=dev)
    new_ts = None
    if gather_timestamps and raw.timestamps is not None:
        new_ts = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    x_out = None
    row = 0
    if x is not None:
        if x.element_size() != 2 or not x.is_cuda or not x.is_contiguous() or x.dim() != 2:
            raise TypeError("x: expected a contiguous 2-d 16-bit device tensor")
        row = int(x.shape[1])
        x_out = torch.empty((max(T, 1), row), dtype=x.dtype, device=dev)
    s = raw.c()
    need = int(lib.hstu_sl_workspace_bytes(ctypes.byref(s)))
    ws = _workspace(need, dev, workspace)
    st = lib.hstu_stochastic_length(ctypes.byref(s), _ptr(u_keep), _ptr(keys), int(n_target),
                                    float(alpha), _ptr(kept), _ptr(new_off), _ptr(new_ts),
                                    _ptr(x), _ptr(x_out), row, _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream))
    _raise(st, "hstu_stochastic_length")
    return kept, new_off, new_ts, x_out


def hstu_layer_bwd_workspace_bytes(dims: LayerDims, seq: DeviceJagged, minimum: bool = False) -> int:
    """Workspace of hstu_layer_bwd: the size that enables the stored-dS path, or with
    minimum=True the least that runs at all."""
    lib = _lib.load()
    d, s = dims.c(), seq.c()
    fn = lib.hstu_layer_bwd_min_workspace_bytes if minimum else lib.hstu_layer_bwd_workspace_bytes
    return int(fn(ctypes.byref(d), ctypes.byref(s)))


def hstu_layer_bwd(dims: LayerDims, w: DeviceWeights, seq: DeviceJagged, x: torch.Tensor,
                   d_y: torch.Tensor, *, bias_grads: bool = True,
                   workspace: Optional[torch.Tensor] = None, stream=None, saved=None):
    """Backward of one causal layer for the upstream gradient d_y (fp32 [T][d]).

    Returns (d_x, grads): d_x fp32 [T][d]; grads a dict of fp32 tensors w1, w2 and, when
    asked for, b1, b2 (bias_grads), and ln_gamma, ln_beta, rab_pos, rab_time for those
    the weights have.  saved: (uvqk, cn, stats) from hstu_layer_fwd_train on the same x and
    weights, to run hstu_layer_bwd_saved instead of recomputing them."""
    lib = _lib.load()
    _check(x, torch.bfloat16, "x")
    _check(d_y, torch.float32, "d_y")
    if saved is not None:
        uvqk, cn, stats = saved
        _check(uvqk, torch.float16, "uvqk")
        _check(cn, torch.float16, "cn")
        _check(stats, torch.float32, "stats")
    dev = x.device
    n1 = dims.uvqk_width
    f32 = dict(dtype=torch.float32, device=dev)
    d_x = torch.empty((seq.total_tokens, dims.d_model), **f32)
    grads = {"w1": torch.empty((n1, dims.d_model), **f32),
             "w2": torch.empty((dims.d_model, dims.hdv), **f32)}
    if bias_grads:
        grads["b1"] = torch.empty(n1, **f32)
        grads["b2"] = torch.empty(dims.d_model, **f32)
    if w.ln_gamma is not None:
        grads["ln_gamma"] = torch.empty(dims.hdv, **f32)
    if w.ln_beta is not None:
        grads["ln_beta"] = torch.empty(dims.hdv, **f32)
    if w.rab_pos is not None:
        grads["rab_pos"] = torch.empty_like(w.rab_pos)
    if w.rab_time is not None:
        grads["rab_time"] = torch.empty_like(w.rab_time)
    gc = _lib.LayerGrads(*(_ptr(grads.get(n)) for n in
                           ("w1", "b1", "w2", "b2", "ln_gamma", "ln_beta", "rab_pos", "rab_time")))
    d, wc, s = dims.c(), w.c(), seq.c()
    need = int(lib.hstu_layer_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(s)))
    ws = _workspace(need, dev, workspace)
    if saved is None:
        st = lib.hstu_layer_bwd(ctypes.byref(d), ctypes.byref(wc), ctypes.byref(s), _ptr(x), _ptr(d_y),
                                _ptr(d_x), ctypes.byref(gc), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream))
        _raise(st, "hstu_layer_bwd")
    else:
        st = lib.hstu_layer_bwd_saved(ctypes.byref(d), ctypes.byref(wc), ctypes.byref(s), _ptr(x),
                                      _ptr(uvqk), _ptr(cn), _ptr(stats), _ptr(d_y), _ptr(d_x),
                                      ctypes.byref(gc), _ptr(ws), ws.numel() * ws.element_size(),
                                      _stream(stream))
        _raise(st, "hstu_layer_bwd_saved")
    return d_x, grads


def hstu_attn_bwd_workspace_bytes(dims: LayerDims, seq: DeviceJagged, minimum: bool = False) -> int:
    """Workspace of hstu_attn_bwd: the size that enables the stored-dS path, or with
    minimum=True the least that runs at all."""
    lib = _lib.load()
    d, s = dims.c(), seq.c()
    fn = lib.hstu_attn_bwd_min_workspace_bytes if minimum else lib.hstu_attn_bwd_workspace_bytes
    return int(fn(ctypes.byref(d), ctypes.byref(s)))


def hstu_attn_bwd(dims: LayerDims, seq: DeviceJagged, q: torch.Tensor, k: torch.Tensor,
                  v: torch.Tensor, d_out: torch.Tensor, *, row_stride: Optional[int] = None,
                  rab_pos: Optional[torch.Tensor] = None, rab_time: Optional[torch.Tensor] = None,
                  rab_grads: bool = False, workspace: Optional[torch.Tensor] = None, stream=None):
    """Gradients of the causal attention for d_out (fp32 [T][H*dv]).  Returns (dq, dk, dv),
    fp32 [T][H*dh] each, and with rab_grads also the gradients of the given bias tables
    (fp32, the tables' shapes; None for a table not given)."""
    lib = _lib.load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.float16 or not t.is_cuda:
            raise TypeError(f"{n}: expected an fp16 device tensor")
    _check(d_out, torch.float32, "d_out")
    if row_stride is None:
        row_stride = q.stride(0)
    T = seq.total_tokens
    dq = torch.empty((T, dims.hdv), dtype=torch.float32, device=q.device)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    d_pos = torch.empty_like(rab_pos) if rab_grads and rab_pos is not None else None
    d_time = torch.empty_like(rab_time) if rab_grads and rab_time is not None else None
    d, s = dims.c(), seq.c()
    need = int(lib.hstu_attn_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(s)))
    ws = _workspace(need, q.device, workspace)
    st = lib.hstu_attn_bwd(ctypes.byref(d), _ptr(rab_pos), _ptr(rab_time), ctypes.byref(s),
                           _ptr(q), _ptr(k), _ptr(v), int(row_stride), _ptr(d_out), _ptr(dq),
                           _ptr(dk), _ptr(dv), _ptr(d_pos), _ptr(d_time), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream(stream))
    _raise(st, "hstu_attn_bwd")
    if rab_grads:
        return dq, dk, dv, d_pos, d_time
    return dq, dk, dv


def hstu_validate_jagged(seq: DeviceJagged, stream=None) -> bool:
    lib = _lib.load()
    s = seq.c()
    st = lib.hstu_validate_jagged(ctypes.byref(s), _stream(stream))
    if st == _lib.HSTU_ERR_INVALID_ARG:
        return False
    _raise(st, "hstu_validate_jagged")
    return True


def profile_enable(on: bool = True, kernels=None):
    """Event timing of the library's launches: every kernel (on=True), none (False), or
    the kernel names in `kernels` (keys of _lib.KERNEL_IDS)."""
    mask = 0
    if on:
        mask = -1 if kernels is None else sum(1 << _lib.KERNEL_IDS[k] for k in kernels)
    _lib.load().hstu_profile_enable(mask)


def profile_reset():
    _lib.load().hstu_profile_reset()


def profile_collect() -> dict:
    """{kernel name: (total ms, launches)} over the records since the last reset."""
    lib = _lib.load()
    tot = (ctypes.c_double * 5)()
    cnt = (ctypes.c_int64 * 5)()
    _raise(lib.hstu_profile_collect(tot, cnt), "hstu_profile_collect")
    return {lib.hstu_kernel_name(i).decode(): (tot[i], cnt[i]) for i in range(5)}


def profile_clock_ghz() -> float:
    """Average shader clock (GHz) over the attention launches made inside a layer while
    profiling was enabled since the last profile_reset, 0.0 if none (include/hstu.h)."""
    lib = _lib.load()
    v = ctypes.c_double(0.0)
    _raise(lib.hstu_profile_clock_ghz(ctypes.byref(v)), "hstu_profile_clock_ghz")
    return float(v.value)
