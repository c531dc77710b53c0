"""ctypes view of libqlin.so (include/qlin.h).  Marshalling only."""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqlin.so")

QLIN_OK = 0
QLIN_FMT_NF4 = 1
QLIN_FMT_INT4_GROUP = 2
QLIN_FMT_NF = 3

#: every symbol include/qlin.h declares
EXPORTS = (
    "qlin_nf4_codebook",
    "qlin_quantize_nf4",
    "qlin_nf_codebook",
    "qlin_quantize_nf",
    "qlin_quantize_int4_group",
    "qlin_workspace_bytes",
    "qlin_fwd",
    "qlin_fwd_noalloc",
    "qlin_bwd",
    "qlin_dequant_bf16",
    "qlin_qa_merge",
    "qlin_int4_scale_zero_grad",
    "qlin_lq_workspace_bytes",
    "qlin_lq_nf4",
    "qlin_profile_next_launch",
    "qlin_status_string",
)


class QWeightStruct(ctypes.Structure):
    _fields_ = [
        ("format", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("dq_block", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("d_out", ctypes.c_int64),
        ("d_in", ctypes.c_int64),
        ("codes", ctypes.c_void_p),
        ("absmax", ctypes.c_void_p),
        ("absmax2", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("zero", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqlin.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m quantized_base_rank_amd.build` "
            "(the layer has no CPU or PyTorch fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    qp = ctypes.POINTER(QWeightStruct)
    sig = {
        "qlin_nf4_codebook": (ctypes.c_int, [vp]),
        "qlin_quantize_nf4": (ctypes.c_int, [vp, i64, i64, i32, i32, vp, vp, vp, vp]),
        "qlin_quantize_int4_group": (ctypes.c_int, [vp, i64, i64, i32, vp, vp, vp, vp]),
        "qlin_nf_codebook": (ctypes.c_int, [i32, vp]),
        "qlin_quantize_nf": (ctypes.c_int, [vp, i64, i64, i32, i32, i32, vp, vp, vp, vp]),
        "qlin_workspace_bytes": (sz, [qp, i64, i32, i32]),
        "qlin_fwd": (ctypes.c_int, [qp, vp, i64, vp, vp, i32, f32, i32, vp, vp, vp, sz, vp]),
        "qlin_fwd_noalloc": (ctypes.c_int, [qp, vp, i64, vp, vp, i32, f32, i32, vp, vp, vp]),
        "qlin_bwd": (ctypes.c_int,
                     [qp, vp, i64, vp, vp, i32, f32, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
        "qlin_dequant_bf16": (ctypes.c_int, [qp, vp, vp]),
        "qlin_profile_next_launch": (ctypes.c_int, [ctypes.c_char_p, vp, vp]),
        "qlin_qa_merge": (ctypes.c_int, [qp, vp, vp, i32, f32, vp, vp]),
        "qlin_int4_scale_zero_grad": (ctypes.c_int, [qp, vp, i64, vp, vp, vp, vp]),
        "qlin_lq_workspace_bytes": (sz, [i64, i64, i32]),
        "qlin_lq_nf4": (ctypes.c_int, [vp, i64, i64, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz,
                                       vp]),
        "qlin_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


class QlinError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().qlin_status_string(status).decode()
        super().__init__(f"{where}: status {status} ({msg})")


def check(status: int, where: str) -> None:
    if status != QLIN_OK:
        raise QlinError(status, where)
