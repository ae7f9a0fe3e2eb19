"""StagQ multi-precision weight-only batch-one GEMV for AMD MI355X (gfx950).

Python face of libstagq.so (C ABI in include/stagq.h).  The functions here only
marshal arguments; packing, decoding and the GEMV run in the native library.

    import precision_weight_only_amd as pwo
    fields = pwo.encode(w_fp16, group=128, nbits=4, budget=K)      # host encoder
    m = pwo.StagQMatrix.pack(fields, device="cuda:0")               # plane-major image in HBM
    y = m.gemv(x_fp16_cuda, bits=3)                                 # precision chosen per call
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, Optional

import numpy as np

from . import _lib as _lib_mod
from ._lib import EXPORTED, Info, StagQError, check, fields_struct, lib  # noqa: F401


def load() -> None:
    """Load libstagq.so now (raises ImportError if it has not been built)."""
    lib()

__all__ = ["StagQMatrix", "encode", "pack_host", "unpack_host", "packed_bytes", "plan_gemv",
           "StagQError"]


def _torch():
    import torch  # PyTorch only provides device memory and streams
    return torch


def _stream_ptr(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def encode(w16: np.ndarray, group: int, nbits: int, budget: int, ratio_T: float = 4.0,
           post_per_row: int = 0) -> Dict:
    """Run the library's host encoder on an fp16 matrix; returns the unpacked
    fields.  post_per_row = k > 0: k post-grid entries per row, budget caps the
    pre-grid guard only."""
    w = np.ascontiguousarray(w16, dtype=np.float16)
    R, Cc = w.shape
    G = Cc // group
    cap = budget + R * post_per_row
    out = dict(
        q=np.empty((R, Cc), np.uint8), planes=np.empty((nbits - 2, R, Cc), np.uint8),
        lo=np.empty((R, G), np.float16), s=np.empty((R, G), np.float16),
        row_ptr=np.empty(R + 1, np.int32), col=np.empty(cap, np.int32),
        val=np.empty(cap, np.float16))
    n_pre = C.c_int64(0)
    p = lambda a: a.ctypes.data_as(C.c_void_p)
    st = lib().stagq_encode(p(w), R, Cc, group, nbits, budget, float(ratio_T), int(post_per_row),
                            p(out["q"]), p(out["planes"]) if nbits > 2 else None, p(out["lo"]),
                            p(out["s"]), p(out["row_ptr"]), p(out["col"]) if cap else None,
                            p(out["val"]) if cap else None, C.byref(n_pre))
    check(st, "stagq_encode")
    nnz = int(out["row_ptr"][-1])
    out["col"], out["val"] = out["col"][:nnz], out["val"][:nnz]
    out.update(group=group, nbits=nbits, n_pre=int(n_pre.value))
    return out


def plan_gemv(rows: int, cols: int, group: int, nbits: int, bits: int, nnz: int = 0,
              side_slots: int = 0) -> Dict[str, int]:
    """Launch shape the library picks for this GEMV (workgroups, threads, ...)."""
    out = (C.c_int32 * 9)()
    check(lib().stagq_plan_gemv(rows, cols, group, nbits, int(nnz), int(side_slots), bits,
                                C.cast(out, C.c_void_p)), "stagq_plan_gemv")
    keys = ("grid", "threads", "waves", "steps_per_wave", "rows_per_group", "lds_bytes",
            "side_wave", "depth", "early_issue")
    return dict(zip(keys, list(out)))


def stream_read(buf, offset: int, nbytes: int, sink, stream=None) -> None:
    """Plain read of nbytes of the uint8 CUDA tensor buf from offset (a
    multiple of 16): the streaming-read ceiling the GEMV is compared with.
    sink: int32 CUDA tensor of one element."""
    if offset % 16 or offset + nbytes > buf.numel():
        raise ValueError("stream_read: offset must be a multiple of 16 and the window inside buf")
    check(lib().stagq_stream_read(C.c_void_p(buf.data_ptr() + offset), int(nbytes),
                                  C.c_void_p(sink.data_ptr()), _stream_ptr(stream)), "stagq_stream_read")


def stream_read_shape(buf, offset: int, nbytes: int, sink, threads: int, loads: int, grid: int = 0,
                      stream=None) -> None:
    """Plain read of nbytes of buf from offset with a chosen launch shape
    (threads per workgroup, 16-byte loads per thread per pass, workgroups;
    grid 0 = one pass): the read-ceiling sweep."""
    if offset % 16 or offset + nbytes > buf.numel():
        raise ValueError("stream_read_shape: offset must be a multiple of 16 and the window inside buf")
    check(lib().stagq_stream_read_shape(C.c_void_p(buf.data_ptr() + offset), int(nbytes),
                                        C.c_void_p(sink.data_ptr()), int(threads), int(loads), int(grid),
                                        _stream_ptr(stream)), "stagq_stream_read_shape")


def check_gemv_args(rows: int, cols: int, device, x, y, x_scale=None) -> None:
    """Raise ValueError (TypeError for non-tensors) unless x is a contiguous fp16
    vector of cols elements, x_scale (if given) likewise, and y a contiguous
    fp32 or fp16 vector of at least rows elements, all on device.  Runs before
    any launch: the library checks only pointers and alignment."""
    torch = _torch()
    for name, t, dtypes, n, exact in (("x", x, (torch.float16,), cols, True),
                                      ("x_scale", x_scale, (torch.float16,), cols, True),
                                      ("y", y, (torch.float32, torch.float16), rows, False)):
        if t is None and name == "x_scale":
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"gemv: {name} must be a torch tensor")
        if t.dtype not in dtypes:
            raise ValueError(f"gemv: {name} must be {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
        if (t.numel() != n) if exact else (t.numel() < n):
            raise ValueError(f"gemv: {name} has {t.numel()} elements, needs {'exactly' if exact else 'at least'} {n}")
        if not t.is_contiguous():
            raise ValueError(f"gemv: {name} must be contiguous")
        if t.device != device:
            raise ValueError(f"gemv: {name} is on {t.device}, the image on {device}")


def _size_error(fs) -> None:
    """stagq_packed_bytes gave 0: raise the status validation reports (the
    packer validates before it looks at its destination)."""
    st = int(lib().stagq_pack_host(C.byref(fs), None, 0))
    check(st if st not in (0, -1) else -3, "stagq_packed_bytes")


def packed_bytes(fields, side_slots: int = 0) -> int:
    keep: list = []
    return int(lib().stagq_packed_bytes(C.byref(fields_struct(fields, keep, side_slots))))


def pack_host(fields, side_slots: int = 0) -> np.ndarray:
    """Packed image in host memory (uint8 array).  side_slots: 0 CSR side
    record, W > 0 fixed slots per row, -1 as many as the fullest row."""
    keep: list = []
    fs = fields_struct(fields, keep, side_slots)
    n = int(lib().stagq_packed_bytes(C.byref(fs)))
    if n == 0:
        _size_error(fs)
    img = np.zeros(n, dtype=np.uint8)
    check(lib().stagq_pack_host(C.byref(fs), img.ctypes.data_as(C.c_void_p), n), "stagq_pack_host")
    return img


def unpack_host(image: np.ndarray) -> Dict:
    """Inverse of pack_host (layout round trip)."""
    image = np.ascontiguousarray(image, dtype=np.uint8)
    info = Info()
    check(lib().stagq_unpack_host(image.ctypes.data_as(C.c_void_p), image.size, C.byref(info),
                                  None, None, None, None, None, None, None), "stagq_unpack_host")
    R, Cc, g, N, nnz = info.rows, info.cols, info.group, info.nbits_max, info.nnz
    out = dict(q=np.empty((R, Cc), np.uint8), planes=np.empty((N - 2, R, Cc), np.uint8),
               lo=np.empty((R, Cc // g), np.uint16), s=np.empty((R, Cc // g), np.uint16),
               row_ptr=np.empty(R + 1, np.int32), col=np.empty(nnz, np.int32),
               val=np.empty(nnz, np.uint16))
    p = lambda a: a.ctypes.data_as(C.c_void_p) if a.size else None
    check(lib().stagq_unpack_host(image.ctypes.data_as(C.c_void_p), image.size, C.byref(info),
                                  p(out["q"]), p(out["planes"]), p(out["lo"]), p(out["s"]),
                                  p(out["row_ptr"]), p(out["col"]), p(out["val"])), "stagq_unpack_host")
    out["lo"] = out["lo"].view(np.float16)
    out["s"] = out["s"].view(np.float16)
    out["val"] = out["val"].view(np.float16)
    out.update(rows=R, cols=Cc, group=g, nbits=N, nnz=nnz, codebook=int(info.codebook),
               side_slots=int(info.side_slots))
    return out


class StagQMatrix:
    """A packed StagQ matrix resident in device memory (one image, every precision)."""

    def __init__(self, handle: C.c_void_p, buffer, info: Info):
        self._h = handle
        self.buffer = buffer          # torch uint8 tensor holding the image (kept alive)
        self.rows, self.cols = info.rows, info.cols
        self.group, self.nbits = info.group, info.nbits_max
        self.nnz = info.nnz
        self.image_bytes = info.image_bytes
        self.bytes_read = {b: int(info.bytes_read[b]) for b in range(2, self.nbits + 1)}
        self.codebook = bool(info.codebook)    # codebook metadata (else fp16 pairs)
        self.side_slots = int(info.side_slots)  # fixed side-record slots per row (0: CSR)

    @classmethod
    def pack(cls, fields, device="cuda:0", stream=None, side_slots: int = 0) -> "StagQMatrix":
        """side_slots: 0 CSR side record, W > 0 fixed slots per row, -1 as
        many as the fullest row."""
        torch = _torch()
        keep: list = []
        fs = fields_struct(fields, keep, side_slots)
        n = int(lib().stagq_packed_bytes(C.byref(fs)))
        if n == 0:
            _size_error(fs)
        buf = torch.empty(n, dtype=torch.uint8, device=device)
        h = C.c_void_p()
        with torch.cuda.device(buf.device):
            check(lib().stagq_pack(C.byref(fs), C.c_void_p(buf.data_ptr()), n, _stream_ptr(stream),
                                   C.byref(h)), "stagq_pack")
        info = Info()
        check(lib().stagq_query(h, C.byref(info)), "stagq_query")
        return cls(h, buf, info)

    def plan(self, bits: int) -> Dict[str, int]:
        """Launch shape of this matrix's GEMV at precision bits."""
        return plan_gemv(self.rows, self.cols, self.group, self.nbits, bits, self.nnz, self.side_slots)

    def clone_to(self, buffer) -> "StagQMatrix":
        """Handle for another device buffer holding a copy of this image."""
        h = C.c_void_p()
        check(lib().stagq_rebind(self._h, C.c_void_p(buffer.data_ptr()), buffer.numel(), C.byref(h)),
              "stagq_rebind")
        info = Info()
        check(lib().stagq_query(h, C.byref(info)), "stagq_query")
        return StagQMatrix(h, buffer, info)

    def replicate(self) -> "StagQMatrix":
        torch = _torch()
        buf = torch.empty_like(self.buffer)
        buf.copy_(self.buffer)
        return self.clone_to(buf)

    def gemv(self, x, bits: int, y=None, stream=None, x_scale=None, out_dtype=None):
        """y = W_hat^(bits) x for an fp16 device vector x; returns fp32 y, or
        fp16 y (stagq_gemv_f16) when out_dtype or the given y is torch.float16.
        x_scale: optional fp16 device vector [cols] of inverse AWQ scales, applied
        to x as it is staged (stagq_gemv_scaled)."""
        torch = _torch()
        if y is None:
            y = torch.empty(self.rows, dtype=out_dtype or torch.float32, device=self.buffer.device)
        check_gemv_args(self.rows, self.cols, self.buffer.device, x, y, x_scale)
        if y.dtype == torch.float16:
            check(lib().stagq_gemv_f16(self._h, C.c_void_p(x.data_ptr()),
                                       C.c_void_p(x_scale.data_ptr()) if x_scale is not None else None,
                                       C.c_void_p(y.data_ptr()), int(bits), _stream_ptr(stream)),
                  "stagq_gemv_f16")
        elif x_scale is None:
            check(lib().stagq_gemv(self._h, C.c_void_p(x.data_ptr()), C.c_void_p(y.data_ptr()),
                                   int(bits), _stream_ptr(stream)), "stagq_gemv")
        else:
            check(lib().stagq_gemv_scaled(self._h, C.c_void_p(x.data_ptr()), C.c_void_p(x_scale.data_ptr()),
                                          C.c_void_p(y.data_ptr()), int(bits), _stream_ptr(stream)),
                  "stagq_gemv_scaled")
        return y

    def gemv_raw(self, x_ptr: int, y_ptr: int, bits: int, stream_ptr) -> int:
        """Launch with raw device pointers; returns the status (no checking)."""
        return lib().stagq_gemv(self._h, C.c_void_p(x_ptr), C.c_void_p(y_ptr), int(bits), stream_ptr)

    def decode_codes(self, bits: int, out=None, stream=None):
        torch = _torch()
        if out is None:
            out = torch.empty((self.rows, self.cols), dtype=torch.uint8, device=self.buffer.device)
        if out.dtype != torch.uint8 or out.numel() < self.rows * self.cols or not out.is_contiguous() \
                or out.device != self.buffer.device:
            raise ValueError("decode_codes: out must be a contiguous uint8 tensor of at least rows * cols "
                             "elements on the image's device")
        check(lib().stagq_decode_codes(self._h, int(bits), C.c_void_p(out.data_ptr()),
                                       _stream_ptr(stream)), "stagq_decode_codes")
        return out

    def __del__(self):
        h = getattr(self, "_h", None)
        try:
            if h and _lib_mod._lib is not None:
                _lib_mod._lib.stagq_destroy(h)
        except Exception:       # interpreter shutdown: modules already torn down
            pass
        self._h = None
