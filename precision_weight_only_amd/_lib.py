"""ctypes binding of the StagQ C ABI (include/stagq.h).

Argument marshalling only: every step of the GEMV runs in libstagq.so.  PyTorch
supplies device memory and streams.  Importing this module fails loudly when the
library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libstagq.so")

STATUS = {
    0: "STAGQ_OK", -1: "STAGQ_EINVAL", -2: "STAGQ_EBITS", -3: "STAGQ_ESHAPE", -4: "STAGQ_ECSR",
    -5: "STAGQ_EALIGN", -6: "STAGQ_EHIP", -7: "STAGQ_EFIELD", -8: "STAGQ_ESIZE", -9: "STAGQ_EIMAGE",
}


class StagQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({lib().stagq_strerror(status).decode()})")


class Codebook(C.Structure):
    _fields_ = [("idx", C.c_void_p), ("log2s", C.c_void_p), ("ratio", C.c_void_p)]


class Fields(C.Structure):
    _fields_ = [
        ("rows", C.c_int32), ("cols", C.c_int32), ("group", C.c_int32), ("nbits_max", C.c_int32),
        ("q", C.c_void_p), ("planes", C.c_void_p), ("lo", C.c_void_p), ("s", C.c_void_p),
        ("row_ptr", C.c_void_p), ("col", C.c_void_p), ("val", C.c_void_p), ("nnz", C.c_int64),
        ("codebook", C.c_void_p), ("side_slots", C.c_int32),
    ]


class Info(C.Structure):
    _fields_ = [
        ("rows", C.c_int32), ("cols", C.c_int32), ("group", C.c_int32), ("nbits_max", C.c_int32),
        ("nnz", C.c_int64), ("image_bytes", C.c_uint64), ("bytes_read", C.c_uint64 * 9),
        ("codebook", C.c_int32), ("side_slots", C.c_int32),
    ]


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m precision_weight_only_amd.build`.  "
            "There is no fallback path.")
    lib = C.CDLL(LIB_PATH)
    P = C.c_void_p
    sig = {
        "stagq_packed_bytes": (C.c_size_t, [C.POINTER(Fields)]),
        "stagq_pack_host": (C.c_int, [C.POINTER(Fields), P, C.c_size_t]),
        "stagq_pack": (C.c_int, [C.POINTER(Fields), P, C.c_size_t, P, C.POINTER(P)]),
        "stagq_rebind": (C.c_int, [P, P, C.c_size_t, C.POINTER(P)]),
        "stagq_gemv": (C.c_int, [P, P, P, C.c_int, P]),
        "stagq_gemv_scaled": (C.c_int, [P, P, P, P, C.c_int, P]),
        "stagq_gemv_f16": (C.c_int, [P, P, P, P, C.c_int, P]),
        "stagq_decode_codes": (C.c_int, [P, C.c_int, P, P]),
        "stagq_query": (C.c_int, [P, C.POINTER(Info)]),
        "stagq_destroy": (None, [P]),
        "stagq_strerror": (C.c_char_p, [C.c_int]),
        "stagq_encode": (C.c_int, [P, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int64,
                                   C.c_double, C.c_int32, P, P, P, P, P, P, P, C.POINTER(C.c_int64)]),
        "stagq_unpack_host": (C.c_int, [P, C.c_size_t, C.POINTER(Info), P, P, P, P, P, P, P]),
        "stagq_plan_gemv": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int64, C.c_int32,
                                      C.c_int, P]),
        "stagq_stream_read": (C.c_int, [P, C.c_size_t, P, P]),
        "stagq_stream_read_shape": (C.c_int, [P, C.c_size_t, P, C.c_int, C.c_int, C.c_int, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = None

# Every symbol the header declares (checked by the CPU test suite).
EXPORTED = (
    "stagq_packed_bytes", "stagq_pack_host", "stagq_pack", "stagq_rebind", "stagq_gemv",
    "stagq_decode_codes", "stagq_query", "stagq_destroy", "stagq_strerror", "stagq_encode",
    "stagq_unpack_host", "stagq_plan_gemv", "stagq_stream_read", "stagq_gemv_scaled",
    "stagq_gemv_f16", "stagq_stream_read_shape",
)


def lib() -> C.CDLL:
    """The loaded library (loaded on first use; raises if it was never built)."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def check(status: int, what: str) -> None:
    if status != 0:
        raise StagQError(status, what)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p) if a is not None and a.size else None


def fields_struct(f, keep: list, side_slots: int = 0) -> Fields:
    """Marshal an unpacked field set (attributes or mapping: rows, cols, group,
    nbits, q, planes, lo, s, row_ptr, col, val) into the C struct.  Arrays are
    converted to the C layout and appended to `keep` so they outlive the call.
    side_slots: 0 CSR side record, W > 0 fixed slots per row, -1 as many as the
    fullest row."""
    get = (lambda k: f[k]) if isinstance(f, dict) else (lambda k: getattr(f, k))
    q = np.ascontiguousarray(get("q"), dtype=np.uint8)
    R, Cc = q.shape
    planes = np.ascontiguousarray(get("planes"), dtype=np.uint8)
    lo = np.ascontiguousarray(np.asarray(get("lo"), dtype=np.float16).view(np.uint16))
    s = np.ascontiguousarray(np.asarray(get("s"), dtype=np.float16).view(np.uint16))
    row_ptr = np.ascontiguousarray(get("row_ptr"), dtype=np.int32)
    col = np.ascontiguousarray(get("col"), dtype=np.int32)
    val = np.ascontiguousarray(np.asarray(get("val"), dtype=np.float16).view(np.uint16))
    nbits = int(get("nbits")) if not isinstance(f, dict) or "nbits" in f else planes.shape[0] + 2
    group = int(get("group"))
    keep.extend([q, planes, lo, s, row_ptr, col, val])
    cb = None
    opt = (lambda k: f.get(k)) if isinstance(f, dict) else (lambda k: getattr(f, k, None))
    if opt("idx") is not None:           # codebook metadata (idx, cb_log2s, cb_ratio)
        idx = np.ascontiguousarray(opt("idx"), dtype=np.uint8)
        l2s = np.ascontiguousarray(np.asarray(opt("cb_log2s"), dtype=np.float16).view(np.uint16))
        rat = np.ascontiguousarray(np.asarray(opt("cb_ratio"), dtype=np.float16).view(np.uint16))
        cb = Codebook(_ptr(idx), _ptr(l2s), _ptr(rat))
        keep.extend([idx, l2s, rat, cb])
    return Fields(R, Cc, group, nbits, _ptr(q), _ptr(planes), _ptr(lo), _ptr(s),
                  row_ptr.ctypes.data_as(C.c_void_p), _ptr(col), _ptr(val), int(col.shape[0]),
                  C.cast(C.pointer(cb), C.c_void_p) if cb is not None else None, int(side_slots))
