"""Pins of the CPU oracle against facts the StagQ paper and mathematics fix.

None of these tests compares the oracle with itself: each expected value is a
number printed in the paper (Figure 1), a hand-worked encoding, a closed form
that differs from the oracle's own formulation, a textbook routine written
inline, or an exact-rational brute force.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import synth_matrix

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _fields_from_codes(q, planes, lo, s, group, mask=None, P=None):
    """Assemble oracle Fields from explicit fields (no encoder involved)."""
    q = np.asarray(q, dtype=np.uint8)
    R, C = q.shape
    planes = np.asarray(planes, dtype=np.uint8).reshape(-1, R, C)
    mask = np.zeros((R, C), bool) if mask is None else np.asarray(mask, bool)
    rr, cc = np.nonzero(mask)
    row_ptr = np.concatenate([[0], np.cumsum(np.bincount(rr, minlength=R))]).astype(np.int32)
    val = np.zeros(0, np.float16) if P is None else np.asarray(P, np.float16)[rr, cc]
    return oracle.Fields(R, C, group, planes.shape[0] + 2, q, planes,
                         np.asarray(lo, np.float16), np.asarray(s, np.float16), mask,
                         row_ptr, cc.astype(np.int32), val)


# ---------------------------------------------------------------- Figure 1
def test_figure1_worked_example():
    g = _load("figure1.json")
    q, bits = oracle.quantize_value(g["w"], g["lo"], g["s"], g["nbits"])
    assert q == g["q"] and bits == g["planes"]


def test_figure1_codes_are_bit_concatenation():
    """Section 3.3: the two bits of q followed by b3..bM form the integer u_M."""
    g = _load("figure1.json")
    F = _fields_from_codes([[g["q"]] * 128], [[[b] * 128] for b in g["planes"]],
                           [[g["lo"]]], [[g["s"]]], 128)
    for M in range(2, g["nbits"] + 1):
        digits = format(g["q"], "02b") + "".join(str(b) for b in g["planes"][:M - 2])
        assert int(oracle.codes(F, M)[0, 0]) == int(digits, 2)


def test_figure1_each_plane_halves_the_spacing():
    """Figure 1: every precision is a uniform grid; each plane halves the spacing,
    so the reconstruction error of 2.15 is at most the half-step t_M (Eq. 7)."""
    g = _load("figure1.json")
    F = _fields_from_codes([[g["q"]] * 128], [[[b] * 128] for b in g["planes"]],
                           [[g["lo"]]], [[g["s"]]], 128)
    for M in range(2, g["nbits"] + 1):
        err = abs(oracle.w_main(F, M)[0, 0] - g["w"])
        assert err <= g["s"] / 2 ** (M - 1) + 1e-15


# ----------------------------------------------------- hand-worked encodes
@pytest.mark.parametrize("case", _load("encoder_small.json")["cases"], ids=lambda c: c["name"])
def test_encoder_hand_worked(case):
    w = np.array(case["w"], dtype=np.float16)
    F = oracle.encode(w, case["group"], case["nbits"], case["frac"], case["T"])
    assert F.q.tolist() == case["q"]
    assert F.planes.tolist() == case["planes"]
    assert F.lo.astype(np.float64).tolist() == case["lo"]
    assert F.s.astype(np.float64).tolist() == case["s"]
    assert F.row_ptr.tolist() == case["row_ptr"]
    assert F.col.tolist() == case["col"]
    assert F.val.astype(np.float64).tolist() == case["val"]
    assert (F.n_pre, F.n_post) == (case["n_pre"], case["n_post"])


# ------------------------------------------------ Eq. 9 against Eq. 10
def _eq9_exact(lo, s, q, bits, M):
    return lo + s * q + sum((2 * b - 1) * s / Fraction(2) ** (k - 1)
                            for k, b in zip(range(3, M + 1), bits))


@pytest.mark.parametrize("N", [2, 3, 4, 5, 6, 7, 8])
def test_eq10_affine_collapse_equals_eq9_exhaustively(N):
    """Section 3.4: lo + s q + sum(2b_k-1) s/2^(k-1) == lo_M + s_M u_M for every
    field combination and every M, in exact rationals; and the oracle's float64
    Eq. (9) equals the exact value."""
    lo, s = Fraction(-3, 7), Fraction(5, 11)
    loM = lambda M: lo - s * (2 ** (M - 2) - 1) / Fraction(2) ** (M - 1)
    sM = lambda M: s / Fraction(2) ** (M - 2)
    n = 4 * 2 ** (N - 2)
    qs = np.array([[c >> (N - 2) for c in range(n)]], dtype=np.uint8)
    planes = np.array([[[(c >> (N - k)) & 1 for c in range(n)]] for k in range(3, N + 1)],
                      dtype=np.uint8).reshape(N - 2, 1, n)
    lo16, s16 = np.float16(-0.4287), np.float16(0.4546)
    F = _fields_from_codes(qs, planes, [[lo16]], [[s16]], n)
    for M in range(2, N + 1):
        u = oracle.codes(F, M)[0]
        wm = oracle.w_main(F, M)[0]
        for c in range(n):
            bits = [int(planes[k - 3, 0, c]) for k in range(3, M + 1)]
            assert _eq9_exact(lo, s, int(qs[0, c]), bits, M) == loM(M) + sM(M) * int(u[c])
            exact16 = _eq9_exact(Fraction(float(lo16)), Fraction(float(s16)), int(qs[0, c]), bits, M)
            assert Fraction(float(wm[c])) == exact16


def test_affine_pair_matches_eq10_closed_form():
    for M in range(2, 9):
        loM, sM = oracle.affine_pair(1.25, 0.75, M)
        assert Fraction(loM) == Fraction(1.25) - Fraction(0.75) * (2 ** (M - 2) - 1) / 2 ** (M - 1)
        assert Fraction(sM) == Fraction(0.75) / 2 ** (M - 2)
        assert oracle.half_step(0.75, M) == sM / 2


# ------------------------------------------- prefix property and midpoints
@pytest.fixture(scope="module")
def tiny_fields():
    w, x = synth_matrix(64, 256, "normal_outliers", 3)
    return oracle.encode(w, 64, 6, 0.01), w, x


def test_prefix_property(tiny_fields):
    """Section 3.3 / Figure 3: a shallower read is the deeper stream truncated."""
    F, _, _ = tiny_fields
    uN = oracle.codes(F, F.nbits).astype(np.int64)
    for M in range(2, F.nbits + 1):
        assert np.array_equal(oracle.codes(F, M), (uN >> (F.nbits - M)).astype(np.uint8))


def test_midpoint_reconstruction(tiny_fields):
    """Section 2.1 and Appendix C (Eq. 12): a shallower read reconstructs at the
    midpoint of the two cells it merges."""
    F, _, _ = tiny_fields
    G = F.cols // F.group
    for M in range(2, F.nbits):
        for r in range(0, F.rows, 7):
            for j in range(G):
                lo, s = float(F.lo[r, j]), float(F.s[r, j])
                loM, sM = oracle.affine_pair(lo, s, M)
                loN, sN = oracle.affine_pair(lo, s, M + 1)
                for u in range(2 ** M):
                    assert loM + sM * u == 0.5 * ((loN + sN * 2 * u) + (loN + sN * (2 * u + 1)))


# ------------------------------------------------------- error bounds
def test_half_step_and_reach_bounds(tiny_fields):
    """Eq. 7: an in-range main-stream entry is within t_M of its weight after M
    bits; Eq. 6: planes move the base reconstruction by at most rho."""
    F, w, _ = tiny_fields
    w = w.astype(np.float64)
    lo = np.repeat(F.lo.astype(np.float64), F.group, axis=1)
    s = np.repeat(F.s.astype(np.float64), F.group, axis=1)
    inside = (~F.mask) & (w >= lo - s / 2) & (w < lo + 3.5 * s)
    assert inside.mean() > 0.9
    base = oracle.w_main(F, 2)
    for M in range(2, F.nbits + 1):
        wm = oracle.w_main(F, M)
        assert np.all(np.abs(w - wm)[inside] <= (s / 2 ** (M - 1))[inside])
        rho = s * (0.5 - 2.0 ** (1 - M))
        assert np.all(np.abs(wm - base) <= rho + 0.0)


def test_closed_form_codes_on_dyadic_inputs():
    """u_N = clamp(floor((w - lo + s/2) 2^(N-2) / s), 0, 2^N - 1): the fine grid's
    cell index, derived from Eq. 8-10 (half-open cells, ties upward)."""
    rng = np.random.default_rng(11)
    N = 6
    mism = 0
    for _ in range(20000):
        s = Fraction(int(rng.integers(1, 64)), 16)
        lo = Fraction(int(rng.integers(-64, 64)), 16)
        # dyadic w, including exact cell boundaries (ties) and out-of-range values
        w = lo + Fraction(int(rng.integers(-40, 4 * 2 ** (N - 2) * 4 + 40)), 4 * 2 ** (N - 2)) * s / 4 * 4
        q, bits = oracle.quantize_value(float(w), float(lo), float(s), N)
        u = int(format(q, "02b") + "".join(map(str, bits)), 2)
        t = (w - lo + s / 2) * 2 ** (N - 2) / s
        want = min(max(t.numerator // t.denominator, 0), 2 ** N - 1)
        mism += (u != want)
    assert mism == 0


# --------------------------------------------------------- side record
def test_held_out_entries_reconstruct_exactly(tiny_fields):
    """Eq. 4: at a held-out position the complete reconstruction is the recorded
    value, at every precision (one P serves every M)."""
    F, w, _ = tiny_fields
    assert F.nnz == oracle.budget(0.01, F.rows, F.cols)
    for M in range(2, F.nbits + 1):
        wh = oracle.w_hat(F, M)
        assert np.array_equal(wh[F.mask], w.astype(np.float64)[F.mask])
        assert np.array_equal(wh[~F.mask], oracle.w_main(F, M)[~F.mask])


def test_guard_invariants(tiny_fields):
    F, w, _ = tiny_fields
    w = w.astype(np.float64)
    # planes skip every held-out position (section 3.6)
    assert not np.any(F.planes[:, F.mask])
    # at most one pre-grid entry per group and it is the group's extreme (section 3.5)
    assert F.n_pre + F.n_post == F.nnz
    # post-grid picks are the largest two-bit residuals among the rest
    lo = np.repeat(F.lo.astype(np.float64), F.group, axis=1)
    s = np.repeat(F.s.astype(np.float64), F.group, axis=1)
    r2 = np.abs(w - (lo + s * F.q))
    G = F.cols // F.group
    mag = np.abs(w).reshape(F.rows, G, F.group)
    pre = np.zeros_like(F.mask)
    cnt = F.mask.reshape(F.rows, G, F.group).sum(axis=2)
    for r in range(F.rows):
        for j in range(G):
            m = F.mask[r, j * F.group:(j + 1) * F.group]
            a = np.sort(mag[r, j])[::-1]
            if m.any() and a[0] > 4 * a[1]:
                c = int(np.argmax(mag[r, j]))
                if m[c]:
                    pre[r, j * F.group + c] = True
    assert pre.sum() >= F.n_pre
    assert np.all(cnt <= 1 + F.group)
    rest = ~F.mask
    post = F.mask & ~pre
    if post.any():
        assert r2[post].min() >= r2[rest].max()


def test_zero_budget_is_plain_dequant_gemv():
    w, x = synth_matrix(16, 256, "student_t", 5)
    F = oracle.encode(w, 128, 4, 0.0)
    assert F.nnz == 0
    for M in (2, 3, 4):
        y = oracle.gemv(F, x, M)
        assert np.array_equal(y, oracle.w_main(F, M) @ x.astype(np.float64))


# --------------------------------------------------- textbook INT2 case
def test_m2_is_groupwise_asymmetric_int2_rtn():
    """With nothing held out, the two-bit read is ordinary group-wise asymmetric
    INT2 round-to-nearest with min-max range (scale = range/3, zero point = min)."""
    w, _ = synth_matrix(32, 512, "student_t", 9)
    g = 128
    F = oracle.encode(w, g, 4, 0.0)
    wf = w.astype(np.float64).reshape(32, -1, g)
    mn = wf.min(axis=2, keepdims=True)
    mx = wf.max(axis=2, keepdims=True)
    scale = ((mx - mn) / (2 ** 2 - 1)).astype(np.float16).astype(np.float64)
    zero = mn.astype(np.float16).astype(np.float64)
    qq = np.clip(np.floor((wf - zero) / np.where(scale > 0, scale, 1) + 0.5), 0, 3)
    qq = np.where(scale > 0, qq, 0)
    deq = (zero + scale * qq).reshape(32, 512)
    assert np.array_equal(oracle.w_main(F, 2), deq)


# ------------------------------------------- brute force in exact rationals
def test_gemv_against_exact_rational_brute_force():
    """Dense W_hat x in exact rationals (Eq. 4 with Eq. 10 per entry) equals the
    oracle's float64 GEMV to rounding, and equals, exactly, the grouped form
    y_r = sum_groups [s_M sum u x + lo_M sum x] + sum_P (P - W_main) x."""
    w, x = synth_matrix(6, 128, "normal_outliers", 21)
    F = oracle.encode(w, 32, 5, 0.02)
    xs = [Fraction(float(v)) for v in x]
    for M in range(2, 6):
        u = oracle.codes(F, M)
        y = oracle.gemv(F, x, M)
        for r in range(F.rows):
            dense = Fraction(0)
            grouped = Fraction(0)
            for j in range(F.cols // F.group):
                lo, s = Fraction(float(F.lo[r, j])), Fraction(float(F.s[r, j]))
                loM = lo - s * (2 ** (M - 2) - 1) / Fraction(2) ** (M - 1)
                sM = s / Fraction(2) ** (M - 2)
                su = Fraction(0)
                sx = Fraction(0)
                for c in range(j * F.group, (j + 1) * F.group):
                    main = loM + sM * int(u[r, c])
                    val = Fraction(float(w[r, c])) if F.mask[r, c] else main
                    dense += val * xs[c]
                    su += int(u[r, c]) * xs[c]
                    sx += xs[c]
                    if F.mask[r, c]:
                        grouped += (Fraction(float(w[r, c])) - main) * xs[c]
                grouped += sM * su + loM * sx
            assert dense == grouped
            assert abs(float(dense) - y[r]) <= 1e-12 * max(1.0, abs(float(dense)))


# --------------------------------------------------- uniform control (App. D)
def test_uniform_control_centroids_sit_at_cell_midpoints():
    """Appendix D: on uniform data the conditional centroid of every interior
    cell sits at the cell midpoint (delta_u = 1/2) at every precision.  The paper
    measures 0.4992..0.5007 on ~10^8 entries; with 2^22 entries here the check is
    |delta_u - 1/2| <= max(0.0008, 5 standard errors)."""
    rng = np.random.default_rng(7)
    g, N = 32, 6
    w = rng.uniform(-1.0, 1.0, size=(1024, 4096))
    F = oracle.encode(w, g, N, 0.0)
    G = w.shape[1] // g
    wg = w.reshape(-1, G, g)
    mn = wg.min(axis=2, keepdims=True)
    mx = wg.max(axis=2, keepdims=True)
    interior_entry = (wg > mn) & (wg < mx)
    lo = F.lo.astype(np.float64)[..., None]
    s = F.s.astype(np.float64)[..., None]
    for M in range(2, N + 1):
        u = oracle.codes(F, M).reshape(-1, G, g).astype(np.int64)
        loM, sM = oracle.affine_pair(lo, s, M)
        a = loM + sM * u - sM / 2                           # lower cell edge
        whole = (a >= mn) & (a + sM <= mx) & interior_entry  # cell wholly inside the range
        pos = ((wg - a) / sM)[whole]
        uu = u[whole]
        for code in np.unique(uu):
            p = pos[uu == code]
            if p.size < 1000:
                continue
            d = p.mean()
            tol = max(0.0008, 5 * 0.2887 / np.sqrt(p.size))
            assert abs(d - 0.5) <= tol, (M, code, d, p.size)


def test_scale_x_rounds_the_exact_product_to_nearest_even():
    """Reading R8 on hand-worked fp16 products: (1 + 2^-10)^2 = 1 + 2^-9 + 2^-20
    rounds down to 1 + 2^-9; (1 + 2^-10) * 1.5 = 1.5 + 1.5 * 2^-10 is a tie
    between 1.5 + 2^-10 (odd) and 1.5 + 2^-9 (even); 2^-14 * 0.5 is the exact
    subnormal 2^-15; 65504 * 2 overflows to +inf; -3 * 0.25 = -0.75."""
    x = np.array([1 + 2 ** -10, 1 + 2 ** -10, 2 ** -14, 65504.0, -3.0], dtype=np.float16)
    a = np.array([1 + 2 ** -10, 1.5, 0.5, 2.0, 0.25], dtype=np.float16)
    want = [1.001953125, 1.501953125, 2.0 ** -15, np.inf, -0.75]
    with np.errstate(over="ignore"):
        got = oracle.scale_x(x, a)
    assert got.dtype == np.float16
    assert [float(v) for v in got] == want


def test_gemv_scaled_special_cases(tiny_fields):
    """Unit scale gives the plain GEMV bitwise; a uniform factor 2 scales y by
    exactly 2; one channel scaled by 3 changes y by that column of W_hat times
    the change of that one activation (so the scale acts on input channels)."""
    F, _, x = tiny_fields
    for M in (2, 4):
        y = oracle.gemv(F, x, M)
        assert np.array_equal(oracle.gemv_scaled(F, x, np.ones(F.cols, np.float16), M), y)
        assert np.array_equal(oracle.gemv_scaled(F, x, np.full(F.cols, 2.0, np.float16), M), 2.0 * y)
        c = 37
        a = np.ones(F.cols, np.float16)
        a[c] = 3.0
        dx = float(np.float16(3.0 * float(x[c]))) - float(x[c])
        col = oracle.w_hat(F, M)[:, c]
        assert np.allclose(oracle.gemv_scaled(F, x, a, M) - y, col * dx, rtol=1e-12, atol=1e-12)


def test_initial_pair_is_symmetric_with_outer_levels_6pct_in():
    """Appendix B / reading R9 on a hand-worked group range [-1, 3]: outer levels
    at -0.76 and 2.76 (6% of the range 4 in from either end), centre level
    midpoint 1.0 = (min + max) / 2, step 0.88 * 4 / 3."""
    lo0, s0 = oracle.initial_pair(-1.0, 3.0)
    assert np.isclose(lo0, -0.76, rtol=0, atol=1e-15)
    assert np.isclose(s0, 3.52 / 3.0, rtol=0, atol=1e-15)
    assert np.isclose(lo0 + 3 * s0, 2.76, rtol=0, atol=1e-14)
    assert np.isclose(lo0 + 1.5 * s0, 1.0, rtol=0, atol=1e-14)


def test_uniform_codebooks_span_the_initial_pairs():
    """Uniform placement: 16 entries from the smallest to the largest log2 s0
    and lo0/s0, equally spaced (s0 = 0 groups ignored).  With log2 s0 in
    {-6, -3} the entries are -6 + i/5 (fp16); with lo0/s0 in {-2, 1} they are
    -2 + i/5."""
    s0 = np.array([2.0 ** -6, 2.0 ** -3, 0.0])
    lo0 = np.array([-2.0 * 2.0 ** -6, 1.0 * 2.0 ** -3, 5.0])
    cs, cr = oracle.uniform_codebooks(lo0, s0)
    assert cs.dtype == np.float16 and cr.dtype == np.float16
    assert [float(v) for v in cs] == [float(np.float16(-6 + i / 5)) for i in range(16)]
    assert [float(v) for v in cr] == [float(np.float16(-2 + i / 5)) for i in range(16)]
    assert float(cs[0]) == -6.0 and float(cs[15]) == -3.0 and float(cs[5]) == -5.0


def test_codebook_table_hand_worked():
    """Reading R10 on hand-worked entries: index i * 16 + j holds
    s = fp16(2^c_s[i]), lo = fp16(c_r[j] * s).  2^-6 = 0.015625 exactly and
    -1.5 * 2^-6 = -0.0234375; 2^-4.5 = 0.0441941738... rounds to
    1448 / 2^15 = 0.044189453125, and -1.5 times that is -1086 / 2^14, exact."""
    cs = np.zeros(16, np.float16); cr = np.zeros(16, np.float16)
    cs[0], cs[1] = -6.0, -4.5
    cr[0], cr[1] = -1.5, 0.25
    lo, s = oracle.codebook_table(cs, cr)
    assert (float(s[0]), float(lo[0])) == (0.015625, -0.0234375)
    assert (float(s[1]), float(lo[1])) == (0.015625, 0.00390625)
    assert (float(s[16]), float(lo[16])) == (0.044189453125, -1086 / 2 ** 14)
    assert (float(s[17]), float(lo[17])) == (0.044189453125, float(np.float16(0.25 * 0.044189453125)))


def _exact_pair_loss(vals, lo, s, N, lam=4):
    """Eq. (5) with E_c = 1 in exact rationals, written independently: nearest
    base level (ties up), each plane the sign of the prefix residual (0 -> +),
    squared errors averaged over M = 2..N, plus lam times the floor term."""
    lo, s = Fraction(lo), Fraction(s)
    rho = s * sum(Fraction(1, 2 ** (k - 1)) for k in range(3, N + 1))
    tot, floor = Fraction(0), Fraction(0)
    for v in vals:
        v = Fraction(v)
        q = 0 if s == 0 else min(3, max(0, sum(1 for j in range(3) if v - lo >= (j + Fraction(1, 2)) * s)))
        rec = lo + s * q
        floor += max(abs(v - rec) - rho, Fraction(0)) ** 2
        tot += (v - rec) ** 2
        for k in range(3, N + 1):
            step = s / 2 ** (k - 1)
            rec = rec + step if v - rec >= 0 else rec - step
            tot += (v - rec) ** 2
    return tot / (N - 1) + lam * floor


@pytest.mark.parametrize("frac", [0.0, 0.02])
def test_codebook_choice_matches_exact_brute_force(frac):
    """The per-group index minimizes Eq. (5) over all 256 pairs, checked in
    exact rationals (lowest index among equal minima); the pre-grid entry, if
    any, enters the loss clamped to the range of the group's other entries."""
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((3, 16)) * 0.05).astype(np.float16)
    w[1, 3] = np.float16(0.9)                      # a pre-grid candidate (ratio > 4)
    N, g = 3, 8
    F = oracle.encode(w, g, N, frac, pair_fit="codebook")
    tlo, ts = oracle.codebook_table(F.cb_log2s, F.cb_ratio)
    assert np.array_equal(F.lo.view(np.uint16), tlo[F.idx].view(np.uint16))
    assert np.array_equal(F.s.view(np.uint16), ts[F.idx].view(np.uint16))
    assert F.n_post == 0 and F.n_pre == (1 if frac else 0)   # K = 1: the one pre-grid entry
    pre = F.mask
    for r in range(3):
        for gi in range(2):
            vals = [float(v) for v in w[r, gi * g:(gi + 1) * g]]
            keep = [v for v, m in zip(vals, pre[r, gi * g:(gi + 1) * g]) if not m]
            vals = [min(max(v, min(keep)), max(keep)) for v in vals]
            losses = [_exact_pair_loss(vals, float(tlo[c]), float(ts[c]), N) for c in range(256)]
            best = min(losses)
            assert losses[int(F.idx[r, gi])] == best
            assert int(F.idx[r, gi]) == losses.index(best)


def test_per_row_post_grid_pick_by_brute_force():
    """encode(..., post_per_row=k): the pre-grid guard takes at most the budget
    (ratio criterion), then every row holds out the k entries with the largest
    |w - (lo + s q)| among those left, lowest column first on ties; written out
    row by row in plain Python against the stored pairs and codes."""
    w, _ = synth_matrix(12, 256, "normal_outliers", 21)
    k = 3
    F = oracle.encode(w, 64, 4, 0.005, post_per_row=k)
    K = oracle.budget(0.005, 12, 256)
    assert 0 < F.n_pre <= K and F.n_post == 12 * k
    assert F.nnz == F.n_pre + F.n_post
    # the pre-grid entries: the ratio criterion, ranked by ratio, capped at K
    cands = []
    for r in range(12):
        for gi in range(4):
            seg = [abs(float(v)) for v in w[r, gi * 64:(gi + 1) * 64]]
            j = seg.index(max(seg))
            second = max(seg[:j] + seg[j + 1:])
            if seg[j] > 4 * second:
                cands.append((-(seg[j] / second) if second else -np.inf, r * 256 + gi * 64 + j))
    pre = {flat for _, flat in sorted(cands)[:K]}
    for r in range(12):
        res = []
        for c in range(256):
            if r * 256 + c in pre:
                continue
            lo, s = float(F.lo[r, c // 64]), float(F.s[r, c // 64])
            res.append((abs(float(w[r, c]) - (lo + s * int(F.q[r, c]))), c))
        res.sort(key=lambda t: (-t[0], t[1]))
        want = {c for _, c in res[:k]} | {f - r * 256 for f in pre if f // 256 == r}
        assert set(np.nonzero(F.mask[r])[0].tolist()) == want, r


# ------------------------------------------------------- budget and row blocks
def test_budget_rounds_halves_up_hand_worked():
    """K = round(frac R C) with a half rounded up (the reading the oracle takes
    where the pages give only a fraction): worked by hand on products that are
    exactly k + 1/2 in binary, and on ones that are not."""
    assert oracle.budget(0.25, 2, 5) == 3        # 2.5 -> 3
    assert oracle.budget(0.5, 1, 7) == 4         # 3.5 -> 4
    assert oracle.budget(0.375, 1, 4) == 2       # 1.5 -> 2
    assert oracle.budget(0.125, 4, 1) == 1       # 0.5 -> 1
    assert oracle.budget(0.25, 1, 9) == 2        # 2.25 -> 2
    assert oracle.budget(0.25, 1, 11) == 3       # 2.75 -> 3
    assert oracle.budget(0.0, 64, 64) == 0
    # the encoder holds out exactly that many on a matrix whose budget is a tie
    w = np.array([[0.0, 0.1, 0.2, 0.3, 9.0],
                  [0.5, -0.4, 0.1, 0.05, 0.0]], np.float16)
    F = oracle.encode(w, 5, 4, 0.25)              # 0.25 * 2 * 5 = 2.5 -> 3 entries
    assert F.nnz == 3
    # by hand: the 9.0 is 30x the next largest of its group (pre-grid, T = 4);
    # the remaining two are the largest two-bit residuals of the rest
    assert F.mask[0, 4] and F.n_pre == 1 and F.n_post == 2


def test_row_blocks_past_the_first_against_exact_rationals():
    """gemv() with row blocks smaller than the matrix (blocks starting past row
    0) and w_hat() on a row slice equal the exact-rational reconstruction of
    Eq. 4 with Eq. 10, entry by entry, including rows with side-record entries."""
    w, x = synth_matrix(7, 64, "normal_outliers", 33)
    F = oracle.encode(w, 32, 4, 0.05)
    assert F.nnz > 0 and len(set(np.nonzero(F.mask)[0])) >= 3
    xs = [Fraction(float(v)) for v in x]
    for M in range(2, 5):
        u = oracle.codes(F, M)

        def exact(r, c):
            j = c // F.group
            lo, s = Fraction(float(F.lo[r, j])), Fraction(float(F.s[r, j]))
            main = lo - s * (2 ** (M - 2) - 1) / Fraction(2) ** (M - 1) + s / Fraction(2) ** (M - 2) * int(u[r, c])
            return Fraction(float(w[r, c])) if F.mask[r, c] else main

        for block_rows in (1, 2, 3):
            y = oracle.gemv(F, x, M, block_rows=block_rows)
            for r in range(F.rows):
                yr = sum(exact(r, c) * xs[c] for c in range(F.cols))
                assert abs(float(yr) - y[r]) <= 1e-12 * max(1.0, abs(float(yr)))
        for r0, r1 in ((2, 5), (6, 7), (1, 7)):
            wh = oracle.w_hat(F, M, slice(r0, r1))
            assert wh.shape == (r1 - r0, F.cols)
            for r in range(r0, r1):
                for c in range(F.cols):
                    assert wh[r - r0, c] == float(exact(r, c))
