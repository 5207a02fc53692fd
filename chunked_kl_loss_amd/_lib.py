"""ctypes loader for libkdkl.so (argument marshalling only)."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# KDKL_LIB may point at another build of the same library (e.g. a variant
# compiled with different tuning constants); default: the in-tree build.
LIB_PATH = os.environ.get("KDKL_LIB") or os.path.join(HERE, "libkdkl.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "kdkl.h")

KDKL_F32 = 0
KDKL_BF16 = 1
STATUS = {
    0: "KDKL_OK", 1: "KDKL_ERR_NULL", 2: "KDKL_ERR_SHAPE", 3: "KDKL_ERR_VALUE",
    4: "KDKL_ERR_DTYPE", 5: "KDKL_ERR_WORKSPACE", 6: "KDKL_ERR_OVERFLOW",
    7: "KDKL_ERR_HIP", 8: "KDKL_ERR_ALIGN", 9: "KDKL_ERR_OPTION",
}
ABI_VERSION = 2
NOALLOC_SCRATCH_BYTES = 64 << 20  # KDKL_NOALLOC_SCRATCH_BYTES
KDKL_LOSS_KL = 0
KDKL_LOSS_JSD = 1
KDKL_LOSS_SKL = 2
KDKL_LOSS_SRKL = 3
KDKL_LOSS_TRKL = 4


class KdklError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {load().kdkl_status_string(status).decode()}")


class KernelStat(C.Structure):
    _fields_ = [
        ("name", C.c_char * 48),
        ("launches", C.c_int64),
        ("total_ms", C.c_double),
        ("flops", C.c_double),
        ("bytes", C.c_double),
    ]


class Options(C.Structure):
    """kdkl_options: per-call options of the fused calls (zero = defaults)."""
    _fields_ = [
        ("loss", C.c_int32),
        ("chunks_per_group", C.c_int32),
        ("vocab_slices", C.c_int32),
        ("dh_w_in_place", C.c_int32),
        ("beta", C.c_float),
        ("reserved", C.c_int32 * 3),
    ]


class Plan(C.Structure):
    """kdkl_plan: the blocking the fused calls use."""
    _fields_ = [
        ("chunks_per_group", C.c_int32),
        ("vocab_slices", C.c_int32),
        ("dh_splits", C.c_int32),
        ("dh_w_in_place", C.c_int32),
        ("vocab_tile", C.c_int32),
        ("hidden_tile", C.c_int32),
        ("bf16_main_loop", C.c_int32),
        ("reserved", C.c_int32),
        ("fwd_bytes", C.c_uint64),
        ("bwd_bytes", C.c_uint64),
    ]


_LIB = None
_P = C.c_void_p
_I64 = C.c_int64
_I32 = C.c_int32

SIGNATURES = {
    "kdkl_abi_version": (C.c_int, []),
    "kdkl_status_string": (C.c_char_p, [C.c_int]),
    "kdkl_workspace_size": (C.c_int, [_I64, _I64, _I64, _I32, _I64, C.c_int, C.POINTER(Options),
                                      C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]),
    "kdkl_plan_info": (C.c_int, [_I64, _I64, _I64, _I32, _I64, C.c_int, C.POINTER(Options),
                                 C.POINTER(Plan)]),
    "kdkl_forward": (C.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, C.c_float, _I64,
                               C.c_int, C.POINTER(Options), _P, _P, _P, _P, C.c_size_t, _P]),
    "kdkl_forward_noalloc": (C.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, C.c_float, _I64,
                                       C.c_int, C.POINTER(Options), _P, _P, _P, _P]),
    "kdkl_backward": (C.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, C.c_float, _I64,
                                C.c_int, C.POINTER(Options), _P, _P, _P, _P, C.c_int, _P,
                                C.c_size_t, _P]),
    "kdkl_logits_forward": (C.c_int, [_P, _P, _P, _I64, _I64, _I32, C.c_float, C.c_int,
                                      _P, _P, _P, _P]),
    "kdkl_logits_backward": (C.c_int, [_P, _P, _P, _I64, _I64, _I32, C.c_float, C.c_int,
                                       _P, _P, _P, _P, C.c_size_t, _P]),
    "kdkl_dense_sizes": (C.c_int, [_I64, _I64, _I64, _I32, C.c_int, C.POINTER(C.c_size_t),
                                   C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]),
    "kdkl_dense_forward": (C.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, C.c_float, C.c_int,
                                     _P, _P, _P, _P, C.c_size_t, _P, C.c_size_t, _P]),
    "kdkl_dense_backward": (C.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, C.c_float, C.c_int,
                                      _P, C.c_size_t, _P, _P, _P, C.c_int, _P, C.c_size_t, _P]),
    "kdkl_check_ids": (C.c_int, [_P, _I64, _I32, _I64, _P, _P, C.c_size_t, _P]),
    "kdkl_profile_begin": (C.c_int, []),
    "kdkl_profile_end": (C.c_int, [C.POINTER(KernelStat), C.c_int, C.POINTER(C.c_int)]),
}


def load():
    """Load libkdkl.so; fails loudly when it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} not found: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.kdkl_abi_version() != ABI_VERSION:
            raise ImportError("libkdkl.so ABI version mismatch")
        _LIB = lib
    return _LIB


def check(status: int, what: str):
    if status != 0:
        raise KdklError(status, what)
