"""Host-side checks of the native library (no GPU): exported symbols, the
plane-major packer and its inverse, argument validation, the fp16 rounding of
the encoder, and the library encoder against the oracle encoder (bit-exact)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
import precision_weight_only_amd as pwo
from precision_weight_only_amd import _lib
from workloads import WORKLOADS, synth_matrix

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_header_symbols_are_exported():
    with open(os.path.join(ROOT, "include", "stagq.h")) as f:
        text = f.read()
    code = re.sub(r"/\*.*?\*/", "", text, flags=re.S)          # drop comments
    declared = set(re.findall(r"\b(stagq_[a-z0-9_]+)\s*\(", code))
    assert declared == set(_lib.EXPORTED)
    lib = pwo.lib()
    for name in declared:
        assert getattr(lib, name) is not None


@pytest.mark.parametrize("post_per_row", [0, 3])
@pytest.mark.parametrize("shape", [(256, 512, 64, 4, 0.005), (33, 384, 32, 6, 0.02), (5, 1024, 128, 8, 0.01)])
def test_library_encoder_matches_oracle(shape, post_per_row):
    R, Cc, g, N, frac = shape
    w, _ = synth_matrix(R, Cc, "normal_outliers", 17)
    F = oracle.encode(w, g, N, frac, post_per_row=post_per_row)
    E = pwo.encode(w, g, N, oracle.budget(frac, R, Cc) if post_per_row else F.nnz, post_per_row=post_per_row)
    assert E["n_pre"] == F.n_pre and E["row_ptr"][-1] == F.nnz
    for k in ("q", "planes", "row_ptr", "col"):
        assert np.array_equal(getattr(F, k), E[k]), k
    for k in ("lo", "s", "val"):
        assert np.array_equal(getattr(F, k).view(np.uint16), E[k].view(np.uint16)), k
    assert E["n_pre"] == F.n_pre


def test_library_encoder_matches_oracle_student_t_full_row_width():
    wl = WORKLOADS["attn"]
    w, _ = synth_matrix(512, 4096, wl.dist, 3)
    F = oracle.encode(w, wl.group, wl.nbits, wl.frac)
    E = pwo.encode(w, wl.group, wl.nbits, F.nnz)
    assert all(np.array_equal(getattr(F, k), E[k]) for k in ("q", "planes", "row_ptr", "col"))


def test_fp16_rounding_of_the_step_matches_numpy():
    """The library's float64 -> fp16 conversion (round to nearest even) on values
    built around fp16 rounding boundaries, via one-row groups whose step is the
    value under test: s16 = fp16((max - min) / 3)."""
    rng = np.random.default_rng(5)
    base = rng.uniform(-3, 3, 4000).astype(np.float16).astype(np.float64)
    w = np.zeros((4000, 32), np.float16)
    w[:, 0] = 0
    w[:, 1] = base.astype(np.float16)
    w[:, 2:] = (base[:, None] / 2).astype(np.float16)
    F = oracle.encode(w, 32, 2, 0.0)
    E = pwo.encode(w, 32, 2, 0)
    assert np.array_equal(F.s.view(np.uint16), E["s"].view(np.uint16))


def test_pack_roundtrip_and_size():
    w, _ = synth_matrix(64, 640, "normal_outliers", 2)
    F = oracle.encode(w, 64, 6, 0.01)
    img = pwo.pack_host(F)
    assert img.size == pwo.packed_bytes(F)
    U = pwo.unpack_host(img)
    for k in ("q", "planes", "row_ptr", "col"):
        assert np.array_equal(getattr(F, k), U[k]), k
    for k in ("lo", "s", "val"):
        assert np.array_equal(getattr(F, k).view(np.uint16), U[k].view(np.uint16)), k


def test_plane_major_layout_offsets():
    """A read at precision M touches the first 256 g' + 1024 M bytes of every
    unit (16 rows x 4 tile columns): the group pairs, then the base stream's
    two chunk stretches, then planes 3..N in order of k.  Rows are padded to a
    multiple of 16 and the 128-column tiles of a row to a multiple of 4."""
    w, _ = synth_matrix(13, 256, "student_t", 4)
    F = oracle.encode(w, 128, 6, 0.0)
    img = pwo.pack_host(F)
    hdr = np.frombuffer(img[:256].tobytes(), dtype=np.uint64)
    quads = int(hdr[6]) & 0xffffffff
    off_units, unit_bytes, unit_meta = int(hdr[7]), int(hdr[8]), int(hdr[9])
    assert quads == 1                           # 2 tiles per row padded to 4
    assert unit_meta == 64 * 4                  # one fp16 pair per tile (g = 128)
    assert unit_bytes == unit_meta + 6 * 1024   # base (2 x 1 KB) + planes 3..6
    # Flipping one refinement bit (plane 5, row 3, column 77) changes exactly
    # one byte: in plane 5's stretch of the unit, at slot 3, dword 77 // 32.
    F2 = oracle.Fields(**{**F.__dict__})
    F2.planes = F.planes.copy()
    F2.planes[2, 3, 77] ^= 1
    img2 = pwo.pack_host(F2)
    diff = np.nonzero(img != img2)[0]
    assert diff.size == 1
    o = off_units + unit_meta + 4 * 1024 + 3 * 16 + 2 * 4
    assert o <= diff[0] < o + 4


def test_bytes_read_model():
    F = oracle.encode(synth_matrix(32, 1024, "student_t", 1)[0], 128, 4, 0.001)
    img = pwo.pack_host(F)
    U = pwo.unpack_host(img)
    info = _lib.Info()
    pwo.lib().stagq_unpack_host(img.ctypes.data_as(C.c_void_p), img.size, C.byref(info),
                                None, None, None, None, None, None, None)
    n = 32 * 1024
    for M in (2, 3, 4):
        want = n * M // 8 + 32 * 8 * 4 + 33 * 4 + F.nnz * 8 + 1024 * 2 + 32 * 4   # row_ptr; side entry: one u64
        assert info.bytes_read[M] == want
    assert U["nnz"] == F.nnz


def _bad(F, **over):
    d = dict(F.__dict__)
    d.update(over)
    return oracle.Fields(**d)


def test_validation_errors():
    w, _ = synth_matrix(8, 256, "normal_outliers", 9)
    F = oracle.encode(w, 64, 4, 0.01)
    assert F.nnz > 0
    q = F.q.copy(); q[0, 0] = 4
    cases = {
        -7: [_bad(F, q=q)],
        -4: [_bad(F, row_ptr=np.concatenate([[1], F.row_ptr[1:]]).astype(np.int32)),
             _bad(F, col=np.where(np.arange(F.nnz) == 0, 999, F.col).astype(np.int32))],
    }
    planes = F.planes.copy()
    r = int(np.searchsorted(F.row_ptr, 0, side="right") - 1)
    planes[0, r, F.col[0]] = 1                       # a plane bit at a held-out position
    cases[-7].append(_bad(F, planes=planes))
    for status, fs in cases.items():
        for f in fs:
            with pytest.raises(pwo.StagQError) as e:
                pwo.pack_host(f)
            assert e.value.status == status
    with pytest.raises(pwo.StagQError) as e:
        pwo.pack_host(_bad(F, cols=200, q=F.q[:, :200]))
    assert e.value.status in (-3, -7, -4)


def test_unsupported_shapes():
    for (R, Cc, g, N) in [(4, 100, 50, 4), (4, 256, 16, 4), (4, 256, 128, 9), (4, 256, 128, 1)]:
        assert pwo.lib().stagq_plan_gemv(R, Cc, g, N, 0, 0, 2, (C.c_int32 * 9)()) == -3
    assert pwo.lib().stagq_plan_gemv(4, 256, 128, 4, 0, 0, 5, (C.c_int32 * 9)()) == -2


def test_strerror_covers_every_status():
    for st in range(0, -10, -1):
        assert pwo.lib().stagq_strerror(st).decode() != "unknown status"


def test_launch_plan_shapes():
    """Launch shapes for a 256-CU device (the host-only default): one
    workgroup per 16-row block; the side record on an extra wave except for a
    heavy CSR record (over 128 entries per block on average) on a grid of fewer
    than two blocks per CU at 2 bits; up to 4 bits each wave takes the most
    steps it can (4, as x is staged for at most 4 steps)."""
    def plan(R, Cc, bits, g=128, N=4, nnz=0, slots=0):
        out = (C.c_int32 * 9)()
        assert pwo.lib().stagq_plan_gemv(R, Cc, g, N, nnz, slots, bits, out) == 0
        return dict(grid=out[0], threads=out[1], S=out[2], steps=out[3], side=out[6])
    p2, p4, p5 = plan(14336, 4096, 2), plan(14336, 4096, 4), plan(14336, 4096, 5, N=6)
    assert (p2["grid"], p2["S"], p2["steps"], p2["side"], p2["threads"]) == (896, 2, 4, 1, 192)
    assert (p4["S"], p4["steps"], p4["threads"]) == (2, 4, 192)
    assert (p5["S"], p5["steps"], p5["threads"]) == (3, 3, 256)
    d = plan(4096, 14336, 2)
    assert (d["grid"], d["S"], d["side"], d["threads"]) == (256, 8, 1, 576)   # no side record: light, one wave more
    dh = plan(4096, 14336, 2, nnz=58720)           # 229 entries per block: after the loop,
    assert (dh["S"], dh["side"], dh["threads"]) == (10, 0, 640)   # at most 3 steps per wave
    assert plan(4096, 14336, 2, nnz=32768)["side"] == 1 and plan(4096, 14336, 2, nnz=32769)["side"] == 0
    assert plan(4096, 14336, 3, nnz=58720, slots=30)["side"] == 1
    assert plan(4096, 14336, 3, nnz=58720)["side"] == 1                  # heavy, small grid: 2 bits only
    d6 = plan(5120, 17920, 6, N=6, nnz=183501)     # 320 blocks, 35 groups of four tile columns
    assert (d6["grid"], d6["S"], d6["side"], d6["threads"]) == (320, 9, 1, 640)
    out = (C.c_int32 * 9)()     # (side wave, depth, early issue) at 4 bits
    assert pwo.lib().stagq_plan_gemv(5120, 17920, 128, 6, 183501, 0, 4, out) == 0 and tuple(out[6:9]) == (1, 1, 0)
    assert pwo.lib().stagq_plan_gemv(14336, 4096, 128, 4, 58720, 0, 4, out) == 0 and tuple(out[6:9]) == (1, 1, 1)
    assert pwo.lib().stagq_plan_gemv(4096, 4096, 128, 4, 16777, 0, 4, out) == 0 and tuple(out[6:9]) == (1, 1, 1)
    assert out[2] == 3                              # few blocks per CU, light record: one wave more
    assert pwo.lib().stagq_plan_gemv(14336, 4096, 128, 4, 58720, 0, 2, out) == 0 and tuple(out[6:9]) == (1, 2, 0)
    assert pwo.lib().stagq_plan_gemv(14336, 4096, 128, 4, 58720, 0, 3, out) == 0 and tuple(out[6:9]) == (1, 1, 1)
    assert pwo.lib().stagq_plan_gemv(4096, 14336, 128, 4, 58720, 0, 2, out) == 0 and tuple(out[6:9]) == (0, 2, 0)
    assert pwo.lib().stagq_plan_gemv(5120, 17920, 128, 6, 183501, 0, 2, out) == 0 and tuple(out[6:9]) == (0, 1, 0)
    assert pwo.lib().stagq_plan_gemv(17920, 5120, 128, 6, 183501, 0, 5, out) == 0 and tuple(out[6:9]) == (1, 1, 0)
    assert out[2] == 4                              # many blocks per CU from 5 bits: one wave more than the fewest
    lm = plan(128256, 4096, 3)
    assert (lm["grid"], lm["S"], lm["side"]) == (8016, 2, 1)


def test_stream_read_argument_errors():
    """The streaming-read ceiling validates its arguments on the host before
    any launch (no GPU needed for these)."""
    lib = pwo.lib()
    sink = C.c_void_p(64)
    assert lib.stagq_stream_read(None, 4096, sink, None) == -1           # EINVAL
    assert lib.stagq_stream_read(C.c_void_p(4096), 4096, None, None) == -1
    assert lib.stagq_stream_read(C.c_void_p(4096), 1 << 31, sink, None) == -1
    assert lib.stagq_stream_read(C.c_void_p(4104), 4096, sink, None) == -5  # EALIGN
    assert lib.stagq_stream_read(C.c_void_p(4096), 0, sink, None) == 0       # nothing to read


def test_codebook_metadata_pack_roundtrip_and_bytes():
    """Codebook metadata (the oracle's codebook encoder): the image stores one
    index byte per group plus the 256 pairs once; unpacking gives back the
    pairs the indices select, bit for bit; the GEMV's byte count charges 1 byte
    per group + 1 KB instead of 4 bytes per group."""
    w, _ = synth_matrix(48, 512, "student_t", 8)
    F = oracle.encode(w, 64, 5, 0.01, pair_fit="codebook")
    Fp = oracle.encode(w, 64, 5, 0.01)
    img = pwo.pack_host(F)
    U = pwo.unpack_host(img)
    assert U["codebook"] == 1
    for k in ("q", "planes", "row_ptr", "col"):
        assert np.array_equal(getattr(F, k), U[k]), k
    for k in ("lo", "s", "val"):
        assert np.array_equal(getattr(F, k).view(np.uint16), U[k].view(np.uint16)), k
    info, infop = _lib.Info(), _lib.Info()
    pwo.lib().stagq_unpack_host(img.ctypes.data_as(C.c_void_p), img.size, C.byref(info),
                                None, None, None, None, None, None, None)
    imgp = pwo.pack_host(Fp)
    pwo.lib().stagq_unpack_host(imgp.ctypes.data_as(C.c_void_p), imgp.size, C.byref(infop),
                                None, None, None, None, None, None, None)
    G = 48 * 512 // 64
    for M in range(2, 6):
        assert info.bytes_read[M] - (F.nnz - Fp.nnz) * 8 == infop.bytes_read[M] - 3 * G + 1024


def test_codebook_metadata_validation():
    """lo, s must be the pairs the indices select (else STAGQ_EFIELD), and the
    codebook pointers must be there (else STAGQ_EINVAL)."""
    w, _ = synth_matrix(16, 256, "student_t", 9)
    F = oracle.encode(w, 128, 4, 0.0, pair_fit="codebook")
    bad = oracle.Fields(**{**F.__dict__})
    bad.idx = F.idx.copy()
    bad.idx[0, 0] ^= 1
    with pytest.raises(pwo.StagQError) as e:
        pwo.pack_host(bad)
    assert e.value.status == -7
    bad = oracle.Fields(**{**F.__dict__})
    bad.cb_ratio = np.zeros(0, np.float16)              # a NULL codebook
    with pytest.raises(pwo.StagQError) as e:
        pwo.pack_host(bad)
    assert e.value.status == -1


def test_fixed_slot_side_record_layout_and_bytes():
    """Fixed side-record slots (the pages' per-row slots): with W = the fullest
    row's count the image round-trips to the same CSR; entry k of row r sits at
    entry ((r / 16) W + k) 16 + r mod 16 of the side region with its column in
    bits 48..63, every other slot is zero; the GEMV's byte count charges W * 8
    bytes per row and no row_ptr."""
    w, _ = synth_matrix(40, 384, "normal_outliers", 18)     # 40 rows: a ragged last block
    F = oracle.encode(w, 64, 4, 0.01)
    counts = np.diff(F.row_ptr)
    W = int(counts.max())
    assert W >= 2 and counts.min() < W
    img = pwo.pack_host(F, side_slots=-1)
    assert img.size == pwo.packed_bytes(F, side_slots=-1)
    U = pwo.unpack_host(img)
    assert U["side_slots"] == W
    for k in ("q", "planes", "row_ptr", "col"):
        assert np.array_equal(getattr(F, k), U[k]), k
    for k in ("lo", "s", "val"):
        assert np.array_equal(getattr(F, k).view(np.uint16), U[k].view(np.uint16)), k
    hdr = img[:256].view(np.uint64)
    off_side = int(hdr[11])
    slots = img[off_side:off_side + 48 * W * 8].view(np.uint64)   # 3 blocks of 16 rows
    seen = np.zeros(slots.size, bool)
    for r in range(F.rows):
        for k, e in enumerate(range(F.row_ptr[r], F.row_ptr[r + 1])):
            at = ((r // 16) * W + k) * 16 + r % 16
            assert int(slots[at]) >> 48 == F.col[e]
            seen[at] = True
    assert not slots[~seen].any()
    Wx = W + 3
    img2 = pwo.pack_host(F, side_slots=Wx)
    info, info0 = _lib.Info(), _lib.Info()
    for im, inf in ((img2, info), (pwo.pack_host(F), info0)):
        pwo.lib().stagq_unpack_host(im.ctypes.data_as(C.c_void_p), im.size, C.byref(inf),
                                    None, None, None, None, None, None, None)
    assert info.side_slots == Wx and info0.side_slots == 0
    for M in (2, 3, 4):
        assert info.bytes_read[M] - 40 * Wx * 8 == info0.bytes_read[M] - 41 * 4 - F.nnz * 8


def test_fixed_slot_side_record_validation():
    """Fewer slots than the fullest row, more than 4096, or a negative count
    other than -1 are STAGQ_ECSR; -1 with an empty side record keeps CSR."""
    w, _ = synth_matrix(16, 256, "student_t", 19)
    F = oracle.encode(w, 128, 4, 0.02)
    W = int(np.diff(F.row_ptr).max())
    for bad in (W - 1, 4097, -2):
        with pytest.raises(pwo.StagQError) as e:
            pwo.pack_host(F, side_slots=bad)
        assert e.value.status == -4, bad
        assert pwo.packed_bytes(F, side_slots=bad) == 0
    F0 = oracle.encode(w, 128, 4, 0.0)
    assert pwo.unpack_host(pwo.pack_host(F0, side_slots=-1))["side_slots"] == 0
    assert pwo.unpack_host(pwo.pack_host(F, side_slots=4096))["side_slots"] == 4096
    # a row fuller than the 4096-slot limit cannot go to slots sized for it
    wb, _ = synth_matrix(1, 16384, "student_t", 20)
    Fb = oracle.encode(wb, 128, 4, 0.3)
    assert int(np.diff(Fb.row_ptr).max()) > 4096
    assert pwo.packed_bytes(Fb, side_slots=-1) == 0 and pwo.packed_bytes(Fb) > 0
    with pytest.raises(pwo.StagQError) as e:
        pwo.pack_host(Fb, side_slots=-1)
    assert e.value.status == -4


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU only: --gpus above 1 exits with status 2 and a
    message, before touching any device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_bench_cpu_baseline_fields():
    """The CPU baseline is the oracle timed on the host: the contract's fields,
    a positive rate, the thread count it used, and a sample description."""
    import bench
    cb = bench.cpu_baseline(rows_sample=64, target_s=0.5)
    assert set(cb) == {"value", "unit", "cores", "kind", "sample"}
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s" and cb["value"] > 0 and cb["cores"] >= 1
    assert "64x4096" in cb["sample"]


def test_host_code_under_sanitizers(tmp_path):
    """The library's host encoder, packer and unpacker (no GPU code) run clean
    under AddressSanitizer and UBSan on round trips of CSR and fixed-slot
    images and on malformed fields and images, each rejected with its status
    (tests/native/host_roundtrip.cpp, built here with g++)."""
    import shutil
    import subprocess
    if shutil.which("g++") is None:
        pytest.skip("no g++")
    exe = str(tmp_path / "host_roundtrip")
    csrc = os.path.join(ROOT, "precision_weight_only_amd", "csrc")
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-pthread", "-I", os.path.join(ROOT, "include"), "-I", csrc,
           os.path.join(ROOT, "tests", "native", "host_roundtrip.cpp"), os.path.join(csrc, "stagq_host.cpp"),
           "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if b.returncode != 0 and ("asan" in b.stderr.lower() or "ubsan" in b.stderr.lower()):
        pytest.skip("sanitizer runtime not available: " + b.stderr[-200:])
    assert b.returncode == 0, b.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                       env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert r.stdout.count("round trip ok") == 6 and "all rejected" in r.stdout


def test_gemv_argument_checks_before_launch():
    """The binding rejects a wrong dtype, length, layout or device of x, x_scale
    or y with ValueError before it calls the library (meta tensors: nothing
    here can reach a device)."""
    import torch
    dev = torch.device("meta")
    R, Cc = 48, 256
    x = torch.empty(Cc, dtype=torch.float16, device=dev)
    y = torch.empty(R, dtype=torch.float32, device=dev)
    pwo.check_gemv_args(R, Cc, dev, x, y)                                   # valid: no error
    pwo.check_gemv_args(R, Cc, dev, x, torch.empty(R + 3, dtype=torch.float16, device=dev), x)
    bad = [
        (torch.empty(Cc, dtype=torch.float32, device=dev), y, None),       # x not fp16
        (torch.empty(Cc + 8, dtype=torch.float16, device=dev), y, None),   # x too long
        (torch.empty(Cc - 8, dtype=torch.float16, device=dev), y, None),   # x too short
        (torch.empty(2 * Cc, dtype=torch.float16, device=dev)[::2], y, None),  # x strided
        (torch.empty(Cc, dtype=torch.float16), y, None),                    # x on another device
        (x, torch.empty(R - 1, dtype=torch.float32, device=dev), None),     # y too short
        (x, torch.empty(R, dtype=torch.float64, device=dev), None),         # y not fp32 / fp16
        (x, torch.empty(2 * R, dtype=torch.float32, device=dev)[::2], None),  # y strided
        (x, y, torch.empty(Cc - 8, dtype=torch.float16, device=dev)),       # scale too short
        (x, y, torch.empty(Cc, dtype=torch.float32, device=dev)),           # scale not fp16
    ]
    for xx, yy, ss in bad:
        with pytest.raises(ValueError):
            pwo.check_gemv_args(R, Cc, dev, xx, yy, ss)
    with pytest.raises(TypeError):
        pwo.check_gemv_args(R, Cc, dev, np.zeros(Cc, np.float16), y)


def test_launch_plan_every_width_and_precision():
    """Every shape the packer accepts has a launch plan (cols up to 32768 in
    steps of 128, every group size, N = 8 at every precision, with and without
    a heavy side record): the widest rows apply the side record after the loop
    when the extra wave does not fit."""
    out = (C.c_int32 * 9)()
    for Cc in list(range(128, 32769, 128)):
        for g in (32, 64, 128):
            for bits in (2, 3, 4, 8):
                for nnz in (0, 200 * 64):
                    st = pwo.lib().stagq_plan_gemv(64, Cc, g, 8, nnz, 0, bits, out)
                    assert st == 0, (Cc, g, bits, nnz, st)
                    assert 0 < out[1] <= 1024 and out[5] <= 160 * 1024
    assert pwo.lib().stagq_plan_gemv(64, 32768, 128, 4, 0, 0, 2, out) == 0 and out[6] == 0


def test_stream_read_shape_argument_errors():
    lib = pwo.lib()
    sink = C.c_void_p(64)
    buf = C.c_void_p(4096)
    assert lib.stagq_stream_read_shape(None, 4096, sink, 256, 1, 0, None) == -1
    assert lib.stagq_stream_read_shape(buf, 4096, None, 256, 1, 0, None) == -1
    assert lib.stagq_stream_read_shape(buf, 1 << 31, sink, 256, 1, 0, None) == -1
    for threads, loads, grid in ((32, 1, 0), (1088, 1, 0), (100, 1, 0), (256, 3, 0), (256, 32, 0), (256, 1, -1)):
        assert lib.stagq_stream_read_shape(buf, 4096, sink, threads, loads, grid, None) == -1
    assert lib.stagq_stream_read_shape(C.c_void_p(4104), 4096, sink, 256, 1, 0, None) == -5
    assert lib.stagq_stream_read_shape(buf, 0, sink, 256, 1, 0, None) == 0


def test_bench_line_names_the_headline_shape():
    """The JSON line reports the shape it timed (14336 x 4096) and a roofline
    fraction that is the 4-bit GEMV's algorithmic bytes over its mean time."""
    import types
    import bench
    from workloads import WORKLOADS
    wl = WORKLOADS[bench.HEADLINE[0]]
    mat = [m for m in wl.matrices if m.name == bench.HEADLINE[1]][0]
    args = types.SimpleNamespace(steps=20, warmup=5, mode="graph")
    bytes_alg = {2: 17107716, 3: 24447748, 4: 31787780}
    dur = {2: [6.0] * 20, 3: [7.0] * 20, 4: [8.0] * 20}
    line = bench.make_line(args, mat, wl, dur, bytes_alg, wall=0.03, launches_per_step=63, n_copies=63,
                           ceiling={}, plans={}, nnz=58720, image_bytes=31840256)
    assert (line["config"]["rows"], line["config"]["cols"]) == (14336, 4096)
    assert line["config"]["gemvs_per_step"] == 189
    assert line["roofline"]["achieved"] == round(31787780 / 8.0e-6 / 1e9, 1)
    assert abs(line["roofline"]["frac"] - 31787780 / 8.0e-6 / 1e9 / 8000) < 1e-4
    assert line["value"] == round(sum(bytes_alg.values()) * 63 * 20 / 0.03 / 1e9, 1)


def test_bench_codebook_fields_select_the_oracle_pairs():
    """bench.codebook_fields (the full-size codebook timing workload) builds
    indices whose (lo, s) are exactly the pairs the oracle's codebook table
    (reading R10) gives for those indices, and the packer accepts them."""
    import bench
    import oracle
    from workloads import synth_matrix
    w, _ = synth_matrix(96, 512, "student_t", 3)
    F = oracle.encode(w, 128, 4, 0.01)
    d = dict(q=F.q, planes=F.planes, lo=F.lo, s=F.s, row_ptr=F.row_ptr, col=F.col, val=F.val,
             group=F.group, nbits=F.nbits)
    cb = bench.codebook_fields(d)
    tlo, ts = oracle.codebook_table(cb["cb_log2s"], cb["cb_ratio"])
    assert np.array_equal(tlo[cb["idx"]].view(np.uint16), np.asarray(cb["lo"], np.float16).view(np.uint16))
    assert np.array_equal(ts[cb["idx"]].view(np.uint16), np.asarray(cb["s"], np.float16).view(np.uint16))
    img = pwo.pack_host(cb)
    back = pwo.unpack_host(img)
    assert back["codebook"] == 1
    assert np.array_equal(back["lo"].view(np.uint16), np.asarray(cb["lo"], np.float16).view(np.uint16))


def test_bench_rotation_exceeds_the_infinity_cache():
    """Timed runs cycle through enough image copies that no launch can find its
    bytes in the 256 MB Infinity Cache: the headline's 63 copies at 2 bits hold
    over 1 GB, every shape's rotation holds at least 4 x the cache, and a
    rotation below that is refused."""
    import bench
    assert bench.rotation_copies(1024, 17107716, minimum=6) == 63
    for b in (1229588, 4893772, 17107716, 27426412, 152987852):
        n = bench.rotation_copies(1024, b)
        assert n * b >= 1024 << 20 and n >= 2
    with pytest.raises(ValueError):
        bench.rotation_copies(512, 17107716)


def test_bench_traffic_profile_matches_the_kernel(monkeypatch):
    """The committed FETCH_SIZE / WRITE_SIZE summary was taken on the current
    kernel source (so the bench line reports it), holds a value per headline
    precision within a few percent above the algorithmic bytes, and is ignored
    once the source changes."""
    import bench
    t = bench.read_traffic()
    assert t is not None, "profiles/gemv_14336x4096_traffic.md is stale for stagq_device.hip"
    alg = {2: 17107716, 3: 24447748, 4: 31787780}
    for M, b in alg.items():
        assert 1.0 <= t[M] / b <= 1.05
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.read_traffic() is None
