"""ctypes mirror of include/hstu.h and include/hstu_layer.h, and the loader of libhstu.so.

Argument marshalling only: every step of the operator runs in the HIP library.
If the library is not built this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhstu.so")

HSTU_OK = 0
HSTU_ERR_INVALID_ARG = 1
HSTU_ERR_UNSUPPORTED = 2
HSTU_ERR_WORKSPACE = 3
HSTU_ERR_HIP = 4
HSTU_FP16 = 0
HSTU_BF16 = 1
HSTU_MAX_GROUPS = 64
HSTU_MAX_SPLITS = 128
HSTU_ABI_VERSION = 4
HSTU_RAB_TIME_BUCKETS = 11
HSTU_RAB_MAX_POS = 2048
HSTU_NOALLOC_SCRATCH_BYTES = 32 << 20

HSTU_ACT_NONE = 0
HSTU_ACT_SILU = 1

# every symbol include/*.h declares
EXPORTED = ("hstu_validate_args", "hstu_fwd_workspace_size", "hstu_fwd", "hstu_fwd_splitkv",
            "hstu_fwd_splitkv_noalloc", "hstu_count_visible_pairs", "hstu_status_string", "hstu_last_error",
            "hstu_abi_version",
            "hstu_linear_fwd", "hstu_norm_gate_fwd", "hstu_layer_workspace_size", "hstu_layer_fwd")


class MaskGroupC(ctypes.Structure):
    _fields_ = [("local_len", ctypes.c_int32), ("context_len", ctypes.c_int32),
                ("minfull_len", ctypes.c_int32), ("attn_scale", ctypes.c_float),
                ("max_uih_q", ctypes.c_int32)]


class FwdArgsC(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("batch", ctypes.c_int32), ("nhead", ctypes.c_int32),
                ("hdim_qk", ctypes.c_int32), ("hdim_v", ctypes.c_int32),
                ("jagged", ctypes.c_int32), ("cross", ctypes.c_int32),
                ("seqlen_q", ctypes.c_int32), ("seqlen_kv", ctypes.c_int32),
                ("total_q", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p),
                ("q_tok_stride", ctypes.c_int64), ("k_tok_stride", ctypes.c_int64),
                ("v_tok_stride", ctypes.c_int64), ("o_tok_stride", ctypes.c_int64),
                ("seq_offsets_q", ctypes.c_void_p), ("seq_offsets_kv", ctypes.c_void_p),
                ("num_targets", ctypes.c_void_p),
                ("causal", ctypes.c_int32), ("softmax", ctypes.c_int32),
                ("alpha", ctypes.c_float), ("num_groups", ctypes.c_int32),
                ("groups", ctypes.POINTER(MaskGroupC)), ("lse", ctypes.c_void_p),
                ("schedule", ctypes.c_int32),
                ("rab_timestamps", ctypes.c_void_p), ("rab_time", ctypes.c_void_p),
                ("rab_pos", ctypes.c_void_p), ("rab_pos_len", ctypes.c_int32),
                ("prof_begin", ctypes.c_void_p), ("prof_end", ctypes.c_void_p)]


class LinearArgsC(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("in_features", ctypes.c_int32), ("out_features", ctypes.c_int32),
                ("x", ctypes.c_void_p), ("x_stride", ctypes.c_int64), ("w", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("activation", ctypes.c_int32),
                ("residual", ctypes.c_void_p), ("residual_stride", ctypes.c_int64),
                ("y", ctypes.c_void_p), ("y_stride", ctypes.c_int64)]


class NormGateArgsC(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("rows", ctypes.c_int64), ("width", ctypes.c_int32),
                ("a", ctypes.c_void_p), ("a_stride", ctypes.c_int64), ("u", ctypes.c_void_p),
                ("u_stride", ctypes.c_int64), ("gamma", ctypes.c_void_p), ("beta", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("z", ctypes.c_void_p), ("z_stride", ctypes.c_int64)]


class LayerArgsC(ctypes.Structure):
    _fields_ = [("attn", FwdArgsC), ("d_model", ctypes.c_int32), ("x", ctypes.c_void_p),
                ("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("ln_gamma", ctypes.c_void_p),
                ("ln_beta", ctypes.c_void_p), ("ln_eps", ctypes.c_float), ("w2", ctypes.c_void_p),
                ("b2", ctypes.c_void_p), ("out", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libhstu.so; raises RuntimeError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           "(run recsys_attention_amd.build.build())")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(FwdArgsC)
    lib.hstu_validate_args.argtypes = [P]
    lib.hstu_validate_args.restype = ctypes.c_int
    lib.hstu_fwd_workspace_size.argtypes = [P, ctypes.c_int32]
    lib.hstu_fwd_workspace_size.restype = ctypes.c_size_t
    lib.hstu_fwd.argtypes = [P, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.hstu_fwd.restype = ctypes.c_int
    lib.hstu_fwd_splitkv.argtypes = [P, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p]
    lib.hstu_fwd_splitkv.restype = ctypes.c_int
    lib.hstu_fwd_splitkv_noalloc.argtypes = [P, ctypes.c_int32, ctypes.c_void_p]
    lib.hstu_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.hstu_count_visible_pairs.argtypes = [P, ctypes.c_void_p, ctypes.c_void_p]
    lib.hstu_count_visible_pairs.restype = ctypes.c_int
    lib.hstu_status_string.argtypes = [ctypes.c_int]
    lib.hstu_status_string.restype = ctypes.c_char_p
    lib.hstu_last_error.argtypes = []
    lib.hstu_last_error.restype = ctypes.c_char_p
    lib.hstu_abi_version.argtypes = []
    lib.hstu_abi_version.restype = ctypes.c_int32
    lib.hstu_linear_fwd.argtypes = [ctypes.POINTER(LinearArgsC), ctypes.c_void_p]
    lib.hstu_linear_fwd.restype = ctypes.c_int
    lib.hstu_norm_gate_fwd.argtypes = [ctypes.POINTER(NormGateArgsC), ctypes.c_void_p]
    lib.hstu_norm_gate_fwd.restype = ctypes.c_int
    lib.hstu_layer_workspace_size.argtypes = [ctypes.POINTER(LayerArgsC)]
    lib.hstu_layer_workspace_size.restype = ctypes.c_size_t
    lib.hstu_layer_fwd.argtypes = [ctypes.POINTER(LayerArgsC), ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_void_p]
    lib.hstu_layer_fwd.restype = ctypes.c_int
    if lib.hstu_abi_version() != HSTU_ABI_VERSION:
        raise RuntimeError("libhstu.so ABI version mismatch")
    _lib = lib
    return lib


class HstuError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def check(status: int) -> None:
    """Raise for a non-OK status: ValueError for argument errors, HstuError otherwise."""
    if status == HSTU_OK:
        return
    lib = load()
    name = lib.hstu_status_string(status).decode()
    msg = f"{name}: {lib.hstu_last_error().decode()}"
    if status in (HSTU_ERR_INVALID_ARG, HSTU_ERR_WORKSPACE):
        err = ValueError(msg)
        err.status = status
        raise err
    raise HstuError(status, msg)
