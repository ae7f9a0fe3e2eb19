"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Decoded codes must match the oracle bit for bit; y must be within relative L2
error 1e-3 of the oracle's float64 GEMV (the StagQ GEMV target).  Two stricter
checks guard regressions:

* every row: |y_r - ref_r| <= 256 * 2^-24 * E_r, where E_r sums the magnitudes
  the fp32 path adds up for that row, sum_c (|lo_M| + s_M u_M) |x_c| plus the
  side record's sum (|a| + s 2^(1-M)) |x_c| (a = P - lo - s (q - 1/2)).  Every
  product of an fp16 code and an fp16 x is exact in fp32; each partial sum is
  bounded by E_r, and no row sum goes through more than about 120 roundings
  (32 per accumulator, 12 in sum(x), 8 over a lane's tiles, 4 S + 1 over the
  lane partials with S <= 15), so the factor 256 covers it twice over;
* the whole vector: ||y - ref|| <= 1e-5 * || |W_hat| |x| ||.

The GEMV's own decode is checked code by code too (test_gemv_decode_one_hot):
one-hot x = e_c makes y_r = lo_M + s_M u_M[r, c] (or P at a held-out entry),
from which u_M is recovered exactly.  Every case prints its name before
touching the GPU.
"""
import functools

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, synth_channel_energy, synth_matrix

pytestmark = pytest.mark.gpu

REL_L2_CONTRACT = 1e-3
REL_L2_REGRESSION = 1e-5


def _say(*a):
    print("[gpu]", *a, flush=True)


@pytest.fixture(scope="module")
def pwo():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_weight_only_amd as m   # raises if libstagq.so is missing
    return m


def _to_dev(x16):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x16).view(np.int16)).view(torch.float16).cuda()


def _rel(y, ref):
    return float(np.linalg.norm(y.astype(np.float64) - ref) / max(np.linalg.norm(ref), 1e-300))


def _abs_scale(F, x, M, rows=None):
    """|| |W_hat| |x| ||_2, the natural scale of the rounding error of y."""
    ax = np.abs(np.asarray(x, np.float64))
    out = np.empty(F.rows)
    for r0 in range(0, F.rows, 8192):
        r1 = min(F.rows, r0 + 8192)
        out[r0:r1] = np.abs(oracle.w_hat(F, M, slice(r0, r1))) @ ax
    return float(np.linalg.norm(out))


def _regression_ok(y, ref, F, x, M):
    return float(np.linalg.norm(y.astype(np.float64) - ref)) <= REL_L2_REGRESSION * _abs_scale(F, x, M)


ROW_ROUNDINGS = 256


def _row_scale(F, x, M, block_rows=8192):
    """E_r of every row (see the module docstring), float64."""
    ax = np.abs(np.asarray(x, np.float64))
    out = np.empty(F.rows)
    loM, sM = oracle.affine_pair(F.lo.astype(np.float64), F.s.astype(np.float64), M)
    u = oracle.codes(F, M)
    for r0 in range(0, F.rows, block_rows):
        r1 = min(F.rows, r0 + block_rows)
        sl = slice(r0, r1)
        mag = np.repeat(np.abs(loM[sl]), F.group, axis=1) + np.repeat(sM[sl], F.group, axis=1) * u[sl]
        out[r0:r1] = mag @ ax
    if F.nnz:
        rr = np.repeat(np.arange(F.rows), np.diff(F.row_ptr))
        jj = F.col // F.group
        s = F.s.astype(np.float64)[rr, jj]
        a = F.val.astype(np.float64) - F.lo.astype(np.float64)[rr, jj] - s * (F.q[rr, F.col].astype(np.float64) - 0.5)
        np.add.at(out, rr, (np.abs(a) + s * 2.0 ** (1 - M)) * ax[F.col])
    return out


def _rows_ok(y, ref, F, x, M):
    """Per-row bound; returns (ok, worst ratio of error to bound)."""
    bound = ROW_ROUNDINGS * 2.0 ** -24 * _row_scale(F, x, M) + 1e-30
    ratio = np.abs(np.asarray(y, np.float64) - ref) / bound
    return bool(np.all(ratio <= 1.0)), float(ratio.max())


@functools.lru_cache(maxsize=8)
def _encoded(workload, mname):
    wl = WORKLOADS[workload]
    mat = [m for m in wl.matrices if m.name == mname][0]
    w, x = synth_matrix(mat.rows, mat.cols, wl.dist, mat.seed)
    F = oracle.encode(w, wl.group, wl.nbits, wl.frac, wl.ratio_T, post_per_row=wl.post_per_row)
    return F, x


def _check(pwo, F, x, bits, tag, codes_rows=None, side_slots=0):
    m = pwo.StagQMatrix.pack(F, side_slots=side_slots)
    xd = _to_dev(x)
    for M in bits:
        _say(tag, f"bits={M}", f"shape={F.rows}x{F.cols}", f"g={F.group}", f"nnz={F.nnz}")
        got = m.decode_codes(M)
        want = oracle.codes(F, M)
        if codes_rows is None:
            assert np.array_equal(got.cpu().numpy(), want), f"codes differ at bits={M}"
        else:
            assert np.array_equal(got[codes_rows].cpu().numpy(), want[codes_rows])
        del got
        y = m.gemv(xd, M).cpu().numpy()
        ref = oracle.gemv(F, x, M)
        rel = _rel(y, ref)
        ok_rows, worst = _rows_ok(y, ref, F, x, M)
        _say(tag, f"bits={M} rel_l2={rel:.3e} worst row error / bound = {worst:.2e}")
        assert rel <= REL_L2_CONTRACT
        assert _regression_ok(y, ref, F, x, M)
        assert ok_rows, f"a row is off by {worst:.2f} x its rounding bound"
    return m, xd


FULL = [(wl, m.name) for wl in ("tiny", "attn", "mlp", "phi4_mlp") for m in WORKLOADS[wl].matrices]
SWEEP = [m.name for m in WORKLOADS["layer_sweep"].matrices if m.name != "lm_head"]


@pytest.mark.parametrize("workload,mname", FULL, ids=[f"{a}-{b}" for a, b in FULL])
def test_workload_parity(pwo, workload, mname):
    F, x = _encoded(workload, mname)
    _check(pwo, F, x, WORKLOADS[workload].bits, f"{workload}/{mname}")


@pytest.mark.parametrize("mname", [m.name for m in WORKLOADS["mlp_rows"].matrices])
def test_per_row_workload_csr_and_fixed_slots(pwo, mname):
    """The MLP shapes at full size with 4 post-grid entries per row: the side
    record as CSR and in fixed per-row slots (W = the fullest row), both to
    the parity bar with codes bit-exact."""
    F, x = _encoded("mlp_rows", mname)
    for slots in (0, -1):
        m, _ = _check(pwo, F, x, WORKLOADS["mlp_rows"].bits, f"mlp_rows/{mname} slots={slots}", side_slots=slots)
        assert m.side_slots == (0 if slots == 0 else int(np.diff(F.row_ptr).max()))
        del m


@pytest.mark.parametrize("mname", SWEEP)
def test_layer_sweep_bits_switched_per_call(pwo, mname):
    """One packed stream, the precision switched on every call (2, 3, 4, 2, ...)."""
    import torch
    wl = WORKLOADS["layer_sweep"]
    F, x = _encoded("layer_sweep", mname)
    m = pwo.StagQMatrix.pack(F)
    xd = _to_dev(x)
    refs = {M: oracle.gemv(F, x, M) for M in wl.bits}
    ys = []
    for i in range(9):
        M = wl.bits[i % 3]
        _say(f"layer_sweep/{mname}", f"call {i} bits={M}")
        ys.append((M, m.gemv(xd, M)))
    torch.cuda.synchronize()
    for M, y in ys:
        assert _rel(y.cpu().numpy(), refs[M]) <= REL_L2_CONTRACT
        assert _regression_ok(y.cpu().numpy(), refs[M], F, x, M)
        assert _rows_ok(y.cpu().numpy(), refs[M], F, x, M)[0]
    for M in wl.bits:  # same bits -> bitwise identical results
        same = [y.cpu().numpy() for b, y in ys if b == M]
        for i, s in enumerate(same[1:], 1):
            d = np.nonzero(same[0] != s)[0]
            assert d.size == 0, (f"bits={M}: call {i} differs from call 0 in {d.size} rows, e.g. "
                                 f"{d[:8].tolist()}: {same[0][d[:4]].tolist()} vs {s[d[:4]].tolist()}")


def _tile_rows(F, reps, rows):
    """Fields of a taller matrix whose row r repeats row r % F.rows."""
    idx = np.arange(rows) % F.rows
    counts = np.diff(F.row_ptr)[idx]
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    starts = F.row_ptr[idx]
    sel = np.concatenate([np.arange(a, a + c) for a, c in zip(starts, counts)]) if counts.sum() else np.zeros(0, int)
    return oracle.Fields(rows, F.cols, F.group, F.nbits, F.q[idx], F.planes[:, idx], F.lo[idx], F.s[idx],
                         F.mask[idx], row_ptr, F.col[sel], F.val[sel])


def test_lm_head_own_draw(pwo):
    """The 128256 x 4096 LM head of the layer sweep on its own draw (Student-t,
    seed 7) with the global 0.1% side-record budget, encoded by the oracle:
    codes bit-exact on every row, y to the parity bar and the per-row bound,
    with the precision switched on every call on the one packed image."""
    import torch
    wl = WORKLOADS["layer_sweep"]
    mat = [m for m in wl.matrices if m.name == "lm_head"][0]
    _say("lm_head own draw: synthesis and oracle encode (about two minutes)")
    w, x = synth_matrix(mat.rows, mat.cols, wl.dist, mat.seed)
    F = oracle.encode(w, wl.group, wl.nbits, wl.frac, wl.ratio_T)
    del w
    assert F.nnz == oracle.budget(wl.frac, mat.rows, mat.cols)
    m = pwo.StagQMatrix.pack(F)
    xd = _to_dev(x)
    for M in wl.bits:
        _say("lm_head own draw", f"bits={M} codes")
        got = m.decode_codes(M).cpu().numpy()
        assert np.array_equal(got, oracle.codes(F, M)), f"codes differ at bits={M}"
        del got
    refs = {M: oracle.gemv(F, x, M) for M in wl.bits}
    ys = []
    for i in range(6):
        M = wl.bits[i % 3]
        _say("lm_head own draw", f"call {i} bits={M}")
        ys.append((M, m.gemv(xd, M)))
    torch.cuda.synchronize()
    for M, y in ys:
        yh = y.cpu().numpy()
        rel = _rel(yh, refs[M])
        ok_rows, worst = _rows_ok(yh, refs[M], F, x, M)
        _say("lm_head own draw", f"bits={M} rel_l2={rel:.3e} worst row error / bound = {worst:.2e}")
        assert rel <= REL_L2_CONTRACT
        assert _regression_ok(yh, refs[M], F, x, M)
        assert ok_rows


def _onehot_check(m, F, M, tiles, tag):
    """The GEMV's own decode, code by code: y = W_hat e_c for every column c of
    the given tiles (one launch per column).  With one-hot x every other column
    contributes an exact zero, so y_r = fl(lo_M + s_M u_M[r, c]) where the main
    stream holds (r, c), from which u_M is recovered exactly; a group of step 0
    decodes to lo exactly; a held-out entry gives the recorded P.  Every entry is
    also held to the oracle's reconstruction within a few fp32 roundings."""
    import torch
    cols = np.concatenate([np.arange(t * 128, (t + 1) * 128) for t in tiles])
    n = cols.shape[0]
    X = torch.zeros((n, F.cols), dtype=torch.float16, device="cuda")
    X[torch.arange(n, device="cuda"), torch.from_numpy(cols).cuda()] = 1.0
    Y = torch.empty((n, F.rows), dtype=torch.float32, device="cuda")
    for i in range(n):
        m.gemv(X[i], M, y=Y[i])
    y = Y.cpu().numpy().T.astype(np.float64)                  # [rows, n]
    del X, Y
    return _onehot_verify(F, M, cols, y, tag)


def _onehot_verify(F, M, cols, y, tag):
    """The checks of _onehot_check on y[r, i] = the GEMV's W_hat[r, cols[i]]."""
    j = cols // F.group
    lo = F.lo.astype(np.float64)[:, j]
    s = F.s.astype(np.float64)[:, j]
    loM, sM = oracle.affine_pair(lo, s, M)
    want = oracle.codes(F, M)[:, cols].astype(np.int64)
    held = F.mask[:, cols]
    pos = (~held) & (s > 0)
    u_hat = np.rint((y - loM) / np.where(sM > 0, sM, 1.0))
    bad = np.argwhere(pos & (u_hat != want))
    assert bad.size == 0, (f"{tag} bits={M}: {len(bad)} codes differ, e.g. (row, col) "
                           f"{[(int(r), int(cols[i])) for r, i in bad[:5]]}")
    zero = (~held) & (s == 0)
    assert np.all(y[zero] == lo[zero])
    wh = oracle.w_hat(F, M)[:, cols]
    P = np.where(held, wh, 0.0)
    q = F.q[:, cols].astype(np.float64)
    a = P - lo - s * (q - 0.5)
    mag = np.abs(loM) + sM * want + np.where(held, np.abs(a) + s * 2.0 ** (1 - M), 0.0)
    err = np.abs(y - wh)
    assert np.all(err <= 2.0 ** -21 * mag + 1e-30), f"{tag} bits={M}: an entry is off by {err.max():.3e}"
    return int(pos.sum()), int(held.sum())


ONEHOT = [("mlp", "gate_up"), ("mlp", "down"), ("phi4_mlp", "gate_up"), ("phi4_mlp", "down")]


@pytest.mark.parametrize("workload,mname", ONEHOT, ids=[f"{a}-{b}" for a, b in ONEHOT])
def test_gemv_decode_one_hot(pwo, workload, mname):
    """The full-size MLP and Phi-4 matrices at every precision: the GEMV's own
    decode recovered code by code from one-hot x over every column of the
    first four tiles (every tile-column lane of the first wave), a middle tile
    and the last four (the last wave), so every base dword, field, plane dword
    and quarter of the decode meets the oracle's u_M (Eq. 8)."""
    wl = WORKLOADS[workload]
    F, _ = _encoded(workload, mname)
    T = F.cols // 128
    tiles = sorted(set([0, 1, 2, 3, T // 2] + list(range(T - 4, T))))
    m = pwo.StagQMatrix.pack(F)
    for M in wl.bits:
        _say(f"one-hot {workload}/{mname}", f"bits={M} tiles={tiles}")
        n_codes, n_held = _onehot_check(m, F, M, tiles, f"{workload}/{mname}")
        _say(f"one-hot {workload}/{mname}", f"bits={M}: {n_codes} codes exact, {n_held} held-out entries")


ONEHOT_SMALL = [
    # (rows, cols, group, nbits, frac, dist, seed, codebook)
    (300, 1024, 128, 8, 0.005, "student_t", 4, False),      # every precision 2..8 (planes 3..8)
    (77, 640, 32, 6, 0.02, "normal_outliers", 3, False),   # g = 32: four groups per tile
    (1001, 384, 64, 4, 0.01, "student_t", 2, False),       # g = 64: two groups per tile, ragged rows
    (300, 1024, 64, 7, 0.005, "student_t", 11, True),      # codebook metadata, odd N
]


@pytest.mark.parametrize("case", ONEHOT_SMALL,
                         ids=[f"{c[0]}x{c[1]}g{c[2]}N{c[3]}{'cb' if c[7] else ''}" for c in ONEHOT_SMALL])
def test_gemv_decode_one_hot_groups_and_precisions(pwo, case):
    """The GEMV's own decode code by code (one-hot x over every column) where
    the full-size matrices do not reach: groups of 32 and 64 columns (several
    (lo, s) pairs per tile), every precision up to 8 bits (the plane-pair and
    odd-plane merges of Eq. 8), and codebook metadata (the pair looked up by
    the group's index)."""
    R, Cc, g, N, frac, dist, seed, cb = case
    w, _ = synth_matrix(R, Cc, dist, seed)
    F = oracle.encode(w, g, N, frac)
    if cb:
        F = _codebook_reindex(F)
    m = pwo.StagQMatrix.pack(F)
    tiles = list(range(Cc // 128))
    for M in range(2, N + 1):
        _say(f"one-hot {case}", f"bits={M}")
        _onehot_check(m, F, M, tiles, f"one-hot {case}")


def _codebook_reindex(F):
    """Fields of the same main stream and side record with codebook metadata:
    two 16-entry fp16 codebooks placed uniformly over the fields' log2 s and
    lo / s, the 256 pairs by the oracle's table (reading R10), and per group the
    index of the pair nearest its (lo, s).  Any index is a valid input of the
    GEMV; the oracle decodes the same fields."""
    lo, s = F.lo.astype(np.float64), F.s.astype(np.float64)
    pos = s > 0
    L, Pr = np.log2(s[pos]), lo[pos] / s[pos]
    t = np.arange(16) / 15.0
    cs = (L.min() + t * (L.max() - L.min())).astype(np.float16)
    cr = (Pr.min() + t * (Pr.max() - Pr.min())).astype(np.float16)
    tlo, ts = oracle.codebook_table(cs, cr)
    i = np.abs(np.log2(np.where(pos, s, 2.0 ** -14))[..., None] - cs.astype(np.float64)).argmin(-1)
    sv = ts[i * 16].astype(np.float64)
    jj = np.abs((lo / sv)[..., None] - cr.astype(np.float64)).argmin(-1)
    idx = (i * 16 + jj).astype(np.uint8)
    return oracle.Fields(F.rows, F.cols, F.group, F.nbits, F.q, F.planes, tlo[idx], ts[idx], F.mask,
                         F.row_ptr, F.col, F.val, idx=idx, cb_log2s=cs, cb_ratio=cr)


FULL_VARIANTS = [("mlp", "gate_up"), ("phi4_mlp", "down")]


@pytest.mark.parametrize("workload,mname", FULL_VARIANTS, ids=[f"{a}-{b}" for a, b in FULL_VARIANTS])
def test_full_size_awq_fp16_codebook(pwo, workload, mname):
    """At the sizes the sweep times them (14336 x 4096, N = 4; 5120 x 17920,
    N = 6, every precision): the AWQ-scaled GEMV against the oracle's
    gemv_scaled, the fp16-output GEMV bitwise fp16(y32) and within half an fp16
    ulp plus the per-row bound of the oracle, and codebook metadata (codes
    bit-exact, y to the parity bar)."""
    import torch
    wl = WORKLOADS[workload]
    F, x = _encoded(workload, mname)
    rng = np.random.default_rng(51)
    a = rng.uniform(0.5, 2.0, F.cols).astype(np.float16)
    xs = oracle.scale_x(x, a)
    m = pwo.StagQMatrix.pack(F)
    xd, ad = _to_dev(x), _to_dev(a)
    for M in wl.bits:
        _say(f"full-size awq / fp16 out {workload}/{mname}", f"bits={M}")
        y = m.gemv(xd, M, x_scale=ad).cpu().numpy()
        ref = oracle.gemv(F, xs, M)
        assert _rel(y, ref) <= REL_L2_CONTRACT
        assert _regression_ok(y, ref, F, xs, M)
        assert _rows_ok(y, ref, F, xs, M)[0]
        y32 = m.gemv(xd, M).cpu().numpy()
        y16 = m.gemv(xd, M, out_dtype=torch.float16).cpu().numpy()
        assert np.array_equal(y16.view(np.uint16), y32.astype(np.float16).view(np.uint16))
        ref0 = oracle.gemv(F, x, M)
        bound = 0.5 * np.spacing(np.abs(y16)).astype(np.float64) + \
            ROW_ROUNDINGS * 2.0 ** -24 * _row_scale(F, x, M)
        assert np.all(np.abs(y16.astype(np.float64) - ref0) <= bound)
    del m
    Fc = _codebook_reindex(F)
    _check(pwo, Fc, x, wl.bits, f"full-size codebook {workload}/{mname}")


# ------------------------------------------------------------- edge cases
EDGE = [
    # (rows, cols, group, nbits, frac, dist, seed)
    (1, 128, 128, 4, 0.0, "student_t", 1),        # one row, one tile, no side record
    (1001, 384, 64, 4, 0.01, "student_t", 2),     # ragged rows, 3 tiles per row
    (77, 640, 32, 6, 0.02, "normal_outliers", 3),  # g = 32, 5 tiles, N = 6
    (300, 1024, 128, 8, 0.005, "student_t", 4),    # N = 8: every precision 2..8
    (64, 4096, 128, 4, 0.1, "student_t", 5),       # more entries than one prefetched chunk
    (513, 8320, 64, 5, 0.001, "student_t", 6),     # 65 tiles per row (> one wave)
    (40, 32768, 128, 4, 0.001, "student_t", 7),    # the widest rows: 16 main waves, record after the loop
    (17, 30720, 64, 4, 0.002, "student_t", 8),     # the widest rows that keep the side-record wave (3-4 bits)
    (3, 32768, 32, 6, 0.01, "normal_outliers", 9),  # g = 32, N = 6 at the widest rows, one block
]


@pytest.mark.parametrize("case", EDGE, ids=[f"{c[0]}x{c[1]}g{c[2]}N{c[3]}" for c in EDGE])
def test_edge_shapes(pwo, case):
    R, Cc, g, N, frac, dist, seed = case
    w, x = synth_matrix(R, Cc, dist, seed)
    F = oracle.encode(w, g, N, frac)
    _check(pwo, F, x, range(2, N + 1), f"edge{case}")


def test_degenerate_values(pwo):
    """Constant groups (stored step 0), zero x, fp16 subnormal x, a held-out entry
    in every group."""
    rng = np.random.default_rng(12)
    w = (0.02 * rng.standard_normal((96, 512))).astype(np.float16)
    w[:8] = np.float16(0.5)                     # constant rows -> s = 0
    w[8:16, ::64] = np.float16(3.0)             # an extreme entry in every group
    F = oracle.encode(w, 64, 4, 0.02)
    assert np.all(F.s[:8] == 0)
    for x in (np.zeros(512, np.float16),
              (rng.standard_normal(512) * 1e-6).astype(np.float16),   # mostly subnormal
              rng.standard_normal(512).astype(np.float16)):
        m = pwo.StagQMatrix.pack(F)
        xd = _to_dev(x)
        for M in (2, 3, 4):
            y = m.gemv(xd, M).cpu().numpy()
            ref = oracle.gemv(F, x, M)
            if not np.any(ref):
                assert not np.any(y)
            else:
                assert _rel(y, ref) <= REL_L2_CONTRACT
                assert _regression_ok(y, ref, F, x, M)


def test_empty_matrix(pwo):
    import torch
    F = oracle.encode(np.zeros((0, 256), np.float16), 128, 4, 0.0)
    m = pwo.StagQMatrix.pack(F)
    y = m.gemv(_to_dev(np.ones(256, np.float16)), 3)
    torch.cuda.synchronize()
    assert y.numel() == 0


def test_deterministic(pwo):
    import torch
    F, x = _encoded("tiny", "W")
    m = pwo.StagQMatrix.pack(F)
    xd = _to_dev(x)
    for M in (2, 3, 4):
        a = m.gemv(xd, M).clone()
        b = m.gemv(xd, M).clone()
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_copies_decode_identically(pwo):
    """A rebound copy of the image (as used for cache-cold timing) gives the same y."""
    import torch
    F, x = _encoded("tiny", "W")
    m = pwo.StagQMatrix.pack(F)
    c = m.replicate()
    xd = _to_dev(x)
    for M in (2, 3, 4):
        assert torch.equal(m.gemv(xd, M), c.gemv(xd, M))


def test_error_codes(pwo):
    import torch
    F, x = _encoded("tiny", "W")
    m = pwo.StagQMatrix.pack(F)
    xd = _to_dev(x)
    for bad in (1, 5, 0, -3):
        with pytest.raises(pwo.StagQError) as e:
            m.gemv(xd, bad)
        assert e.value.status == -2
    xbig = torch.zeros(F.cols + 8, dtype=torch.float16, device="cuda")
    with pytest.raises(pwo.StagQError) as e:
        m.gemv(xbig[1:F.cols + 1], 3)            # 2-byte offset: not 16-byte aligned
    assert e.value.status == -5
    with pytest.raises(pwo.StagQError) as e:
        m.decode_codes(7)
    assert e.value.status == -2
    with pytest.raises(pwo.StagQError) as e:
        m.gemv(xd, 3, x_scale=xbig[1:F.cols + 1])   # misaligned scale
    assert e.value.status == -5
    # the binding's own checks, before any launch
    for bad in (xbig, xd.float(), xd.cpu(), torch.zeros(2 * F.cols, dtype=torch.float16, device="cuda")[::2]):
        with pytest.raises(ValueError):
            m.gemv(bad, 3)
    with pytest.raises(ValueError):
        m.gemv(xd, 3, y=torch.empty(F.rows - 1, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        m.gemv(xd, 3, y=torch.empty(F.rows, dtype=torch.float64, device="cuda"))
    assert pwo.lib().stagq_gemv_scaled(m._h, xd.data_ptr(), None, xd.data_ptr(), 3, None) == -1


def test_side_wave_reads_x_from_lds_or_global(pwo, monkeypatch):
    """The side-record wave reads x_c from the x the main waves staged in LDS
    once their flags are up, and from global memory when its spin limit runs
    out first: a spin limit of 0 sends some workgroups down each road, and y
    must be bitwise the same (same x values, same summation order)."""
    monkeypatch.setenv("STAGQ_SIDE", "1")
    w, xe = synth_matrix(2048, 1024, "student_t", 11)
    F = oracle.encode(w, 128, 4, 0.02)
    m, xd = _check(pwo, F, xe, (2, 4), "side wave x source (default spins)")
    ys = {M: m.gemv(xd, M).cpu().numpy() for M in (2, 4)}
    monkeypatch.setenv("STAGQ_FLAG_SPINS", "0")
    for M in (2, 4):
        _say("side wave x source (spin limit 0)", f"bits={M}")
        assert np.array_equal(m.gemv(xd, M).cpu().numpy(), ys[M])


@pytest.mark.parametrize("side", ["0", "1"])
def test_side_record_modes(pwo, side, monkeypatch):
    """Both places the side record can be applied (all waves after the main
    loop, or an extra wave of the workgroup; the library picks one per shape)
    meet the parity bar on small and skewed side records."""
    monkeypatch.setenv("STAGQ_SIDE", side)
    F, x = _encoded("tiny", "W")
    _check(pwo, F, x, (2, 3, 4), f"tiny side={side}")
    for case in ((1001, 384, 64, 4, 0.01, "student_t", 2), (77, 640, 32, 6, 0.02, "normal_outliers", 3),
                 (64, 4096, 128, 4, 0.1, "student_t", 5)):
        R, Cc, g, N, frac, dist, seed = case
        w, xe = synth_matrix(R, Cc, dist, seed)
        _check(pwo, oracle.encode(w, g, N, frac), xe, range(2, N + 1), f"edge{case} side={side}")


def test_stream_read_ceiling_kernel(pwo):
    """The streaming-read ceiling reads and discards: zeros never hit the
    checksum, so sink stays untouched; a ragged byte count is fine."""
    import torch
    _say("stream_read 1 MiB + 48 B of zeros")
    buf = torch.zeros((1 << 20) + 4096, dtype=torch.uint8, device="cuda")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    pwo.stream_read(buf, 16, (1 << 20) + 48, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7


@pytest.mark.parametrize("side", ["0", "1"])
def test_awq_scaled_gemv(pwo, side, monkeypatch):
    """The run-time inverse AWQ scale folded into x staging (stagq_gemv_scaled)
    against the oracle's gemv_scaled on ragged, wide and skewed-side-record
    shapes, in both side-record modes; a unit scale gives the plain GEMV
    bitwise; the side-record wave's global-x fallback scales x_c the same way."""
    import torch
    monkeypatch.setenv("STAGQ_SIDE", side)
    rng = np.random.default_rng(23)
    for case in ((1001, 384, 64, 4, 0.01, "student_t", 2), (2048, 1024, 128, 4, 0.02, "student_t", 11),
                 (64, 4096, 128, 6, 0.1, "normal_outliers", 5)):
        R, Cc, g, N, frac, dist, seed = case
        w, x = synth_matrix(R, Cc, dist, seed)
        F = oracle.encode(w, g, N, frac)
        a = rng.uniform(0.25, 4.0, Cc).astype(np.float16)
        m = pwo.StagQMatrix.pack(F)
        xd, ad = _to_dev(x), _to_dev(a)
        one = _to_dev(np.ones(Cc, np.float16))
        xs = oracle.scale_x(x, a)
        for M in range(2, N + 1):
            _say(f"awq scaled {case} side={side}", f"bits={M}")
            y = m.gemv(xd, M, x_scale=ad).cpu().numpy()
            ref = oracle.gemv_scaled(F, x, a, M)
            assert _rel(y, ref) <= REL_L2_CONTRACT
            assert _regression_ok(y, ref, F, xs, M)
            assert np.array_equal(m.gemv(xd, M, x_scale=one).cpu().numpy(), m.gemv(xd, M).cpu().numpy())
            if side == "1":
                monkeypatch.setenv("STAGQ_FLAG_SPINS", "0")
                assert np.array_equal(m.gemv(xd, M, x_scale=ad).cpu().numpy(), y)
                monkeypatch.delenv("STAGQ_FLAG_SPINS")
        torch.cuda.synchronize()


@pytest.mark.parametrize("side", ["0", "1"])
def test_codebook_metadata_gemv(pwo, side, monkeypatch):
    """The pages' metadata (one codebook index per group, 256 pairs per matrix;
    the oracle's codebook encoder) against the oracle: codes bit-exact, y to the
    parity bar, in both side-record modes, on ragged rows, g = 32 / 64 / 128,
    N = 4 and 6; also with the run-time AWQ scale."""
    monkeypatch.setenv("STAGQ_SIDE", side)
    rng = np.random.default_rng(31)
    for case in ((1001, 384, 64, 4, 0.01, "student_t", 2), (77, 640, 32, 6, 0.02, "normal_outliers", 3),
                 (512, 2048, 128, 4, 0.001, "student_t", 4)):
        R, Cc, g, N, frac, dist, seed = case
        w, x = synth_matrix(R, Cc, dist, seed)
        F = oracle.encode(w, g, N, frac, pair_fit="codebook")
        m, xd = _check(pwo, F, x, range(2, N + 1), f"codebook {case} side={side}")
        assert m.codebook
        a = rng.uniform(0.5, 2.0, Cc).astype(np.float16)
        ad = _to_dev(a)
        for M in (2, N):
            _say(f"codebook {case} side={side} awq", f"bits={M}")
            y = m.gemv(xd, M, x_scale=ad).cpu().numpy()
            ref = oracle.gemv_scaled(F, x, a, M)
            assert _rel(y, ref) <= REL_L2_CONTRACT
            assert _regression_ok(y, ref, F, oracle.scale_x(x, a), M)


@pytest.mark.parametrize("side", ["0", "1"])
def test_fp16_output_gemv(pwo, side, monkeypatch):
    """The fp16-output GEMV (stagq_gemv_f16) rounds the very row sums the fp32
    GEMV writes: bitwise fp16(y32) with and without the AWQ scale and on
    codebook metadata, within half an fp16 ulp plus the fp32 summation bound of
    the oracle's y and to the parity bar; row sums beyond the fp16 range become +-inf exactly where fp16(y32)
    does."""
    import torch
    monkeypatch.setenv("STAGQ_SIDE", side)
    rng = np.random.default_rng(41)
    for case in ((1001, 384, 64, 4, 0.01, "student_t", 2, "minmax"), (77, 640, 32, 6, 0.02, "normal_outliers", 3, "codebook"),
                 (2048, 1024, 128, 4, 0.02, "student_t", 11, "minmax")):
        R, Cc, g, N, frac, dist, seed, fit = case
        w, x = synth_matrix(R, Cc, dist, seed)
        F = oracle.encode(w, g, N, frac, pair_fit=fit)
        m = pwo.StagQMatrix.pack(F)
        a = rng.uniform(0.5, 2.0, Cc).astype(np.float16)
        xd, ad = _to_dev(x), _to_dev(a)
        for M in range(2, N + 1):
            for sc in (None, ad):
                _say(f"fp16 out {case} side={side} awq={sc is not None}", f"bits={M}")
                y32 = m.gemv(xd, M, x_scale=sc).cpu().numpy()
                y16 = m.gemv(xd, M, x_scale=sc, out_dtype=torch.float16).cpu().numpy()
                assert y16.dtype == np.float16
                assert np.array_equal(y16.view(np.uint16), y32.astype(np.float16).view(np.uint16))
                xe = x if sc is None else oracle.scale_x(x, a)
                ref = oracle.gemv(F, xe, M)
                # per row: half an fp16 ulp of rounding plus the fp32 summation
                # error, bounded by 1e-5 of sum |W_hat| |x| as elsewhere
                bound = 0.5 * np.spacing(np.abs(y16)).astype(np.float64) + \
                    REL_L2_REGRESSION * (np.abs(oracle.w_hat(F, M)) @ np.abs(xe.astype(np.float64)))
                assert np.all(np.abs(y16.astype(np.float64) - ref) <= bound)
                assert _rel(y16, ref) <= REL_L2_CONTRACT
    # beyond the fp16 range: large weights and activations
    w, x = synth_matrix(256, 1024, "student_t", 5)
    w = (w.astype(np.float64) * 4000).astype(np.float16)
    x = (x.astype(np.float64) * 30).astype(np.float16)
    F = oracle.encode(w, 128, 4, 0.01)
    m = pwo.StagQMatrix.pack(F)
    xd = _to_dev(x)
    for M in (2, 4):
        _say(f"fp16 out overflow side={side}", f"bits={M}")
        y32 = m.gemv(xd, M).cpu().numpy()
        y16 = m.gemv(xd, M, out_dtype=torch.float16).cpu().numpy()
        with np.errstate(over="ignore"):
            want = y32.astype(np.float16)
        assert np.isinf(want).any() and np.isfinite(want).any()
        assert np.array_equal(y16.view(np.uint16), want.view(np.uint16))
    yodd = torch.empty(F.rows + 1, dtype=torch.float16, device="cuda")
    assert pwo.lib().stagq_gemv_f16(m._h, xd.data_ptr(), None, yodd.data_ptr() + 1, 3, None) == -5
    assert pwo.lib().stagq_gemv_f16(m._h, xd.data_ptr(), None, yodd.data_ptr() + 2, 3, None) == 0
    torch.cuda.synchronize()


@functools.lru_cache(maxsize=8)
def _full_encoded(case, criterion, storage="weight"):
    R, Cc, g, N, dist, seed = case
    w, x = synth_matrix(R, Cc, dist, seed)
    return oracle.encode_full(w, g, N, E=synth_channel_energy(Cc, seed), criterion=criterion, tau=1e-4,
                              storage=storage), x


@pytest.mark.parametrize("criterion", ["ratio", "gain"])
@pytest.mark.parametrize("side", ["0", "1"])
def test_full_encoder_workload(pwo, criterion, side, monkeypatch):
    """The oracle's full encoder as a second workload: codebooks placed by the
    best of the nine rules, E_c-weighted pairs whose levels sit off the group
    extremes, the ratio or gain criterion and per-row post-grid entries.  Codes
    bit-exact and y to the parity bar in both side-record modes, on ragged rows,
    g = 128 and 32, N = 4 and 6."""
    monkeypatch.setenv("STAGQ_SIDE", side)
    for case in ((72, 1024, 128, 4, "student_t", 21), (40, 512, 32, 6, "normal_outliers", 22)):
        F, x = _full_encoded(case, criterion)
        m, _ = _check(pwo, F, x, range(2, case[3] + 1), f"full encoder {criterion} {case} side={side}")
        assert m.codebook
        # the pages' pairing: per-row post-grid picks in fixed per-row slots
        m, _ = _check(pwo, F, x, (2, case[3]), f"full encoder {criterion} {case} side={side} slots",
                      side_slots=-1)
        assert m.side_slots == int(np.diff(F.row_ptr).max())
        # the pages' side-record codes (8-bit pre-grid codes, fp16 residuals)
        Fp, _ = _full_encoded(case, criterion, "paper")
        _check(pwo, Fp, x, (2, case[3]), f"full encoder {criterion} {case} side={side} paper codes")


@pytest.mark.parametrize("side", ["0", "1"])
def test_fixed_slot_side_record(pwo, side, monkeypatch):
    """The side record in fixed per-row slots (no row_ptr on the GEMV's path):
    codes bit-exact and y to the parity bar against the oracle in both
    side-record modes, with W the fullest row's count and with spare slots, on
    ragged rows and on rows of several hundred entries (many slot batches);
    the side-record wave's global-x fallback gives bitwise the same y; with the
    AWQ scale and with an fp16 result too."""
    import torch
    monkeypatch.setenv("STAGQ_SIDE", side)
    rng = np.random.default_rng(43)
    for case in ((256, 512, 64, 4, 0.005, "normal_outliers", 0), (1001, 384, 64, 4, 0.01, "student_t", 2),
                 (64, 4096, 128, 4, 0.1, "normal_outliers", 5), (77, 640, 32, 6, 0.02, "student_t", 3)):
        R, Cc, g, N, frac, dist, seed = case
        w, x = synth_matrix(R, Cc, dist, seed)
        F = oracle.encode(w, g, N, frac)
        W = int(np.diff(F.row_ptr).max())
        for slots in (-1, W + 5):
            tag = f"slots={slots} (fullest row {W}) {case} side={side}"
            m, xd = _check(pwo, F, x, range(2, N + 1), tag, side_slots=slots)
            assert m.side_slots == (W if slots == -1 else slots)
        a = rng.uniform(0.5, 2.0, Cc).astype(np.float16)
        ad = _to_dev(a)
        for M in (2, N):
            _say(f"slots {case} side={side} awq / fp16 out / fallback", f"bits={M}")
            y = m.gemv(xd, M, x_scale=ad).cpu().numpy()
            ref = oracle.gemv_scaled(F, x, a, M)
            assert _rel(y, ref) <= REL_L2_CONTRACT
            assert _regression_ok(y, ref, F, oracle.scale_x(x, a), M)
            y32 = m.gemv(xd, M).cpu().numpy()
            y16 = m.gemv(xd, M, out_dtype=torch.float16).cpu().numpy()
            assert np.array_equal(y16.view(np.uint16), y32.astype(np.float16).view(np.uint16))
            if side == "1":
                monkeypatch.setenv("STAGQ_FLAG_SPINS", "0")
                assert np.array_equal(m.gemv(xd, M).cpu().numpy(), y32)
                assert np.array_equal(m.gemv(xd, M, x_scale=ad).cpu().numpy(), y)
                monkeypatch.delenv("STAGQ_FLAG_SPINS")
