"""ctypes mirror of include/sage.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsage.so")

SAGE_OK = 0
STATUS_NAMES = {
    0: "SAGE_OK", 1: "SAGE_ERR_NULL", 2: "SAGE_ERR_DTYPE", 3: "SAGE_ERR_LAYOUT",
    4: "SAGE_ERR_HEAD_DIM", 5: "SAGE_ERR_SHAPE", 6: "SAGE_ERR_GQA", 7: "SAGE_ERR_STRIDE",
    8: "SAGE_ERR_ALIGN", 9: "SAGE_ERR_WORKSPACE", 10: "SAGE_ERR_SEQLENS", 11: "SAGE_ERR_ARCH",
    12: "SAGE_ERR_HIP", 13: "SAGE_ERR_FLAGS",
}
F16, BF16 = 0, 1
PV_FP8, PV_HALF = 0, 1
PV_MODES = {"fp8": PV_FP8, "half": PV_HALF}
KV_SPLIT_AUTO = -1
HND, NHD = 0, 1
QK_BLOCK, KV_TILE = 64, 128
NOALLOC_WS_MAX = 64 << 20     # SAGE_NOALLOC_WS_MAX

EXPORTS = ["sage_desc_init", "sage_quant_buf_sizes", "sage_workspace_size", "sage_quant_qkv",
           "sage_attn_fwd", "sage_attn_fwd_varlen", "sage_attn_fwd_quantized",
           "sage_attn_fwd_noalloc",
           "sage_debug_qk_int32", "sage_debug_e4m3_encode", "sage_kv_split_size",
           "sage_micro_rate", "sage_status_string", "sage_abi_version"]
MICRO_OPS = {"i8": 0, "f8": 1, "exp": 2, "fma": 3}   # sage_micro_op


class Desc(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("layout", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32), ("nq", ctypes.c_int32),
        ("nkv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("is_causal", ctypes.c_int32), ("smooth_q", ctypes.c_int32),
        ("smooth_k", ctypes.c_int32), ("smooth_v", ctypes.c_int32),
        ("sm_scale", ctypes.c_float), ("pv_mode", ctypes.c_int32),
        ("kv_split", ctypes.c_int32), ("qk_block", ctypes.c_int32),
    ]


_BUF_FIELDS = ["mu_q", "mu_k", "mu_v", "q_codes", "q_scale", "k_codes", "k_scale", "v_codes",
               "v_scale", "delta_s", "mu_qb", "mu_q_code", "mu_q_cscale"]
ABI_VERSION = 3
SMOOTH_Q_BLOCK = 2           # SAGE_SMOOTH_Q_BLOCK


class QuantBufs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _BUF_FIELDS]


class QuantSizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in _BUF_FIELDS]


_lib = None


class LibraryMissing(RuntimeError):
    pass


def lib():
    """Load libsage.so; raise if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(
            f"{LIB_PATH} is missing: build it with `python -m quantized_attention_03_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32 = ctypes.c_void_p, ctypes.c_int32
    D = ctypes.POINTER(Desc)
    ip = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "sage_desc_init": (None, [D, I32, I32, I32, I32, I32, I32, I32, I32]),
        "sage_quant_buf_sizes": (I32, [D, ip, ip, I32, ctypes.POINTER(QuantSizes)]),
        "sage_workspace_size": (I32, [D, ip, ip, I32, ctypes.POINTER(ctypes.c_size_t)]),
        "sage_quant_qkv": (I32, [D, P, P, P, ip, ip, I32, ctypes.POINTER(QuantBufs), P,
                                 ctypes.c_size_t, P]),
        "sage_attn_fwd": (I32, [D, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "sage_attn_fwd_noalloc": (I32, [D, P, P, P, P, P, P]),
        "sage_attn_fwd_varlen": (I32, [D, ip, ip, I32, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "sage_attn_fwd_quantized": (I32, [D, ip, ip, I32, ctypes.POINTER(QuantBufs), P, P, P,
                                          ctypes.c_size_t, P]),
        "sage_kv_split_size": (I32, [D, ip, ip, I32, ip]),
        "sage_debug_qk_int32": (I32, [D, ip, ip, I32, ctypes.POINTER(QuantBufs), P, P]),
        "sage_debug_e4m3_encode": (I32, [ctypes.c_uint32, ctypes.c_uint32, P, P]),
        "sage_micro_rate": (I32, [I32, I32, ctypes.POINTER(ctypes.c_double), P]),
        "sage_status_string": (ctypes.c_char_p, [I32]),
        "sage_abi_version": (I32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    if L.sage_abi_version() != ABI_VERSION:
        raise LibraryMissing(
            f"{LIB_PATH} has ABI version {L.sage_abi_version()}, the binding expects "
            f"{ABI_VERSION}: rebuild it with `python -m quantized_attention_03_amd.build`")
    _lib = L
    return L


class SageError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        name = STATUS_NAMES.get(status, str(status))
        msg = lib().sage_status_string(status).decode()
        super().__init__(f"{fn} failed: {name} ({msg})")


def check(fn: str, status: int) -> None:
    if status != SAGE_OK:
        raise SageError(fn, status)
