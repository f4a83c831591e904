"""ctypes view of include/hstu.h and loader for the in-tree libhstu.so.

Argument marshalling only: structures mirror the C declarations field for field.
The library must have been built (``__graft_entry__.build()`` or ``python -m
hstu_pointwise_attention_jagged_amd.build``); there is no fallback of any kind.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhstu.so")

c_int32, c_int64, c_float, c_double, c_void_p, c_size_t = (
    ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p, ctypes.c_size_t)

HSTU_OK, HSTU_ERR_INVALID_ARG, HSTU_ERR_UNSUPPORTED, HSTU_ERR_WORKSPACE, HSTU_ERR_HIP = range(5)
MASK_CAUSAL, MASK_SELF_ONLY = 0, 1
KERNEL_IDS = {"schedule": 0, "f1_gemm_silu": 1, "attention": 2, "f2_prep": 3, "f2_gemm": 4}


class Dims(ctypes.Structure):
    _fields_ = [("d_model", c_int32), ("num_heads", c_int32), ("dqk", c_int32), ("dv", c_int32),
                ("pos_buckets", c_int32), ("time_buckets", c_int32), ("rab_heads", c_int32),
                ("ln_eps", c_float)]


class Weights(ctypes.Structure):
    _fields_ = [("w1", c_void_p), ("b1", c_void_p), ("w2", c_void_p), ("b2", c_void_p),
                ("ln_gamma", c_void_p), ("ln_beta", c_void_p), ("rab_pos", c_void_p),
                ("rab_time", c_void_p)]


class LayerGrads(ctypes.Structure):
    _fields_ = [("w1", c_void_p), ("b1", c_void_p), ("w2", c_void_p), ("b2", c_void_p),
                ("ln_gamma", c_void_p), ("ln_beta", c_void_p), ("rab_pos", c_void_p),
                ("rab_time", c_void_p)]


class Jagged(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("total_tokens", c_int32), ("max_seq_len", c_int32),
                ("seq_offsets", c_void_p), ("timestamps", c_void_p)]


class Prefix(ctypes.Structure):
    _fields_ = [("seq", ctypes.POINTER(Jagged)), ("k", c_void_p), ("v", c_void_p),
                ("row_stride", c_int64)]


EXPORTS = {
    "hstu_layer_workspace_bytes": (c_size_t, [ctypes.POINTER(Dims), ctypes.POINTER(Jagged)]),
    "hstu_mfalcon_workspace_bytes": (c_size_t, [ctypes.POINTER(Dims), ctypes.POINTER(Jagged),
                                                ctypes.POINTER(Jagged)]),
    "hstu_attn_workspace_bytes": (c_size_t, [ctypes.POINTER(Dims), ctypes.POINTER(Jagged),
                                             ctypes.POINTER(Jagged)]),
    "hstu_layer_fwd": (c_int32, [ctypes.POINTER(Dims), ctypes.POINTER(Weights), ctypes.POINTER(Jagged),
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "hstu_layer_fwd_mfalcon": (c_int32, [ctypes.POINTER(Dims), ctypes.POINTER(Weights),
                                         ctypes.POINTER(Jagged), c_void_p, ctypes.POINTER(Jagged),
                                         c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "hstu_attn_fwd": (c_int32, [ctypes.POINTER(Dims), c_void_p, c_void_p, ctypes.POINTER(Jagged),
                                c_void_p, c_void_p, c_void_p, c_int64, ctypes.POINTER(Prefix),
                                c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "hstu_attn_noalloc_max_scratch_bytes": (c_size_t, []),
    "hstu_attn_fwd_noalloc": (c_int32, [ctypes.POINTER(Dims), c_void_p, c_void_p, ctypes.POINTER(Jagged),
                                        c_void_p, c_void_p, c_void_p, c_int64, ctypes.POINTER(Prefix),
                                        c_int32, c_void_p, c_void_p]),
    "hstu_stack_workspace_bytes": (c_size_t, [ctypes.POINTER(Dims), ctypes.POINTER(Jagged)]),
    "hstu_stack_mfalcon_workspace_bytes": (c_size_t, [ctypes.POINTER(Dims), ctypes.POINTER(Jagged),
                                                      ctypes.POINTER(Jagged)]),
    "hstu_stack_fwd": (c_int32, [ctypes.POINTER(Dims), c_int32, ctypes.POINTER(Weights),
                                 ctypes.POINTER(Jagged), c_void_p, c_void_p, c_void_p, c_int32,
                                 c_void_p, c_size_t, c_void_p]),
    "hstu_stack_fwd_mfalcon": (c_int32, [ctypes.POINTER(Dims), c_int32, ctypes.POINTER(Weights),
                                         ctypes.POINTER(Jagged), c_void_p, ctypes.POINTER(Jagged),
                                         c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "hstu_layer_bwd_workspace_bytes": (c_size_t, [ctypes.POINTER(Dims), ctypes.POINTER(Jagged)]),
    "hstu_layer_bwd_min_workspace_bytes": (c_size_t, [ctypes.POINTER(Dims), ctypes.POINTER(Jagged)]),
    "hstu_attn_bwd_min_workspace_bytes": (c_size_t, [ctypes.POINTER(Dims), ctypes.POINTER(Jagged)]),
    "hstu_layer_bwd": (c_int32, [ctypes.POINTER(Dims), ctypes.POINTER(Weights), ctypes.POINTER(Jagged),
                                 c_void_p, c_void_p, c_void_p, ctypes.POINTER(LayerGrads), c_void_p,
                                 c_size_t, c_void_p]),
    "hstu_layer_fwd_train": (c_int32, [ctypes.POINTER(Dims), ctypes.POINTER(Weights), ctypes.POINTER(Jagged),
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_size_t, c_void_p]),
    "hstu_layer_bwd_saved": (c_int32, [ctypes.POINTER(Dims), ctypes.POINTER(Weights), ctypes.POINTER(Jagged),
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       ctypes.POINTER(LayerGrads), c_void_p, c_size_t, c_void_p]),
    "hstu_attn_bwd_workspace_bytes": (c_size_t, [ctypes.POINTER(Dims), ctypes.POINTER(Jagged)]),
    "hstu_attn_bwd": (c_int32, [ctypes.POINTER(Dims), c_void_p, c_void_p, ctypes.POINTER(Jagged),
                                c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                c_void_p]),
    "hstu_sl_workspace_bytes": (c_size_t, [ctypes.POINTER(Jagged)]),
    "hstu_stochastic_length": (c_int32, [ctypes.POINTER(Jagged), c_void_p, c_void_p, c_int32, c_double,
                                         c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                                         c_void_p, c_size_t, c_void_p]),
    "hstu_validate_jagged": (c_int32, [ctypes.POINTER(Jagged), c_void_p]),
    "hstu_status_str": (ctypes.c_char_p, [c_int32]),
    "hstu_last_hip_error": (ctypes.c_int, []),
    "hstu_profile_enable": (None, [ctypes.c_int]),
    "hstu_profile_reset": (None, []),
    "hstu_profile_collect": (c_int32, [ctypes.POINTER(c_double), ctypes.POINTER(c_int64)]),
    "hstu_kernel_name": (ctypes.c_char_p, [ctypes.c_int]),
    "hstu_profile_clock_ghz": (c_int32, [ctypes.POINTER(c_double)]),
}

_LIB = None


def load(path: str = LIB_PATH):
    """Load libhstu.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the HIP library first "
                           "(python -m hstu_pointwise_attention_jagged_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib
