"""Pins of the oracle's full encoder (codebook placement rules, the weighted
pair choice, the gain criterion of Eq. (11) and the per-row post-grid guard)
against what the StagQ paper and mathematics fix.

Each expected value comes from somewhere other than the encoder's own
vectorised loss: closed forms (cluster means, the bit charge), an exact-rational
loss, the single-value quantizer and decoder reconstructions, or brute force
written out per row and per group in plain Python.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import synth_channel_energy, synth_matrix


# ------------------------------------------------------------------ Lloyd
def _distortion(v, c):
    return float(sum(min((x - y) ** 2 for y in c) for x in v))


def test_lloyd_recovers_separated_cluster_means():
    """Sixteen clusters {k - 1/8, k + 1/8}: Lloyd's rule from the uniform start
    ends on the cluster means k; anchored, the ends stay at the range ends
    (-1/8 and 15 + 1/8) and the fourteen interior centres are the means."""
    v = np.array([k + d for k in range(16) for d in (-0.125, 0.125)])
    c = oracle.place_codebook(v, "lloyd").astype(np.float64)
    assert list(c) == list(range(16))
    a = oracle.place_codebook(v, "lloyd_anchored").astype(np.float64)
    assert a[0] == -0.125 and a[15] == 15.125
    assert list(a[1:15]) == list(range(1, 15))
    u = oracle.place_codebook(v, "uniform").astype(np.float64)
    assert list(u) == [float(np.float16(-0.125 + i * 15.25 / 15)) for i in range(16)]


@pytest.mark.parametrize("anchored", [False, True])
def test_lloyd_distortion_never_rises_and_ends_at_a_fixed_point(anchored):
    """Each round of Lloyd's rule (anchored or not) cannot raise the squared
    distortion; at the end every free centre is the mean of its cell (nearest
    centre, lower one on ties) and the anchored ends are the range ends."""
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(300), 4 + 0.3 * rng.standard_normal(60)])
    init = v.min() + np.arange(16) / 15 * (v.max() - v.min())
    prev = _distortion(v, init)
    for it in range(1, 30):
        c = oracle.lloyd_1d(v, init, anchored=anchored, max_iter=it)
        d = _distortion(v, c)
        assert d <= prev * (1 + 1e-12)
        prev = d
    c = oracle.lloyd_1d(v, init, anchored=anchored)
    cells = [[] for _ in range(16)]
    for x in v:
        dist = [abs(x - y) for y in c]
        cells[dist.index(min(dist))].append(x)
    for k in range(16):
        if anchored and k in (0, 15):
            assert c[k] == init[k]
        elif cells[k]:
            assert math.isclose(c[k], sum(cells[k]) / len(cells[k]), rel_tol=0, abs_tol=1e-12)


# -------------------------------------------------- weighted choice, exact
def _exact_loss(vals, wts, lo, s, N, lam):
    """Eq. (5) with Eq. (6) in exact rationals, weights E_c: nearest base level
    (ties up), planes by the sign of the prefix residual (0 counts +)."""
    lo, s = Fraction(lo), Fraction(s)
    rho = s * sum(Fraction(1, 2 ** (k - 1)) for k in range(3, N + 1))
    tot = floor = Fraction(0)
    for v, e in zip(vals, wts):
        v, e = Fraction(v), Fraction(e)
        q = 0 if s == 0 else sum(1 for j in range(3) if v - lo >= (j + Fraction(1, 2)) * s)
        rec = lo + s * q
        floor += e * max(abs(v - rec) - rho, Fraction(0)) ** 2
        tot += e * (v - rec) ** 2
        for k in range(3, N + 1):
            step = s / 2 ** (k - 1)
            rec = rec + step if v - rec >= 0 else rec - step
            tot += e * (v - rec) ** 2
    return tot / (N - 1) + lam * floor


def test_weighted_pair_choice_matches_exact_brute_force():
    """Every group's index minimizes the E_c-weighted Eq. (5) (lambda = 4) over
    the 256 pairs of the chosen codebooks, checked in exact rationals on the
    group with its pre-grid entry clipped to the range of the others (lowest
    index among equal minima)."""
    w, _ = synth_matrix(2, 32, "normal_outliers", 4)
    w[0, 5] = np.float16(0.75)                     # a pre-grid entry (ratio > 4)
    E = np.array([2.0 ** (i % 5 - 2) for i in range(32)])   # dyadic weights 1/4 .. 4
    N, g = 3, 16
    F = oracle.encode_full(w, g, N, E=E)
    tlo, ts = oracle.codebook_table(F.cb_log2s, F.cb_ratio)
    assert np.array_equal(F.lo.view(np.uint16), tlo[F.idx].view(np.uint16))
    assert F.mask[0, 5]
    for r in range(2):
        for gi in range(2):
            cols = range(gi * g, (gi + 1) * g)
            vals = [float(w[r, c]) for c in cols]
            pre = [c == 5 and r == 0 for c in cols]
            keep = [v for v, p in zip(vals, pre) if not p]
            vals = [min(max(v, min(keep)), max(keep)) for v in vals]
            losses = [_exact_loss(vals, E[gi * g:(gi + 1) * g], float(tlo[c]), float(ts[c]), N, 4)
                      for c in range(256)]
            assert int(F.idx[r, gi]) == losses.index(min(losses))


def test_uniform_weights_scale_out_of_the_choice():
    """Multiplying every E_c by the same power of two changes no choice (the
    loss scales exactly), and E_c = 1 gives the same fields as no E at all."""
    w, _ = synth_matrix(8, 128, "student_t", 6)
    Fa = oracle.encode_full(w, 32, 4)
    Fb = oracle.encode_full(w, 32, 4, E=np.full(128, 8.0))
    Fc = oracle.encode_full(w, 32, 4, E=np.ones(128))
    for F in (Fb, Fc):
        assert np.array_equal(F.idx, Fa.idx) and np.array_equal(F.q, Fa.q)
        assert np.array_equal(F.mask, Fa.mask) and np.array_equal(F.planes, Fa.planes)


# ------------------------------------------------------ rule choice (FE3)
def _first_term_via_quantizer(vals, wts, lo, s, N):
    """First term of Eq. (5) through the single-value quantizer and the
    additive reconstruction of Eq. (9), one value at a time."""
    tot = 0.0
    for v, e in zip(vals, wts):
        q, b = oracle.quantize_value(v, lo, s, N)
        rec = lo + s * q
        tot += e * (v - rec) ** 2
        for k in range(3, N + 1):
            rec += (2 * b[k - 3] - 1) * s / 2.0 ** (k - 1)
            tot += e * (v - rec) ** 2
    return tot / (N - 1)


def test_rule_pair_is_the_brute_force_best_of_nine():
    """The chosen placement rules minimize the matrix's first Eq. (5) term,
    each group taking its best pair under that term, over the nine rule
    combinations; recomputed through the single-value quantizer."""
    w, _ = synth_matrix(2, 64, "student_t", 8)
    E = synth_channel_energy(64, 8)
    N, g = 3, 16
    F = oracle.encode_full(w, g, N, E=E, T=1e9, fallback=np.inf)   # no pre-grid entries, no fallback
    assert F.n_pre == 0 and not F.info["fell_back"]
    wg = w.astype(np.float64).reshape(2, 4, g)
    lo0, s0 = oracle.initial_pair(wg.min(axis=2), wg.max(axis=2))
    L, P = np.log2(s0).ravel(), (lo0 / s0).ravel()
    scores = {}
    for rs in ("uniform", "lloyd", "lloyd_anchored"):
        for rr in ("uniform", "lloyd", "lloyd_anchored"):
            tlo, ts = oracle.codebook_table(oracle.place_codebook(L, rs), oracle.place_codebook(P, rr))
            tot = 0.0
            for r in range(2):
                for gi in range(4):
                    vals = [float(v) for v in wg[r, gi]]
                    tot += min(_first_term_via_quantizer(vals, E[gi * g:(gi + 1) * g], float(tlo[c]),
                                                         float(ts[c]), N) for c in range(256))
            scores[(rs, rr)] = tot
    best = min(scores.values())
    first = [k for k, v in scores.items() if v <= best * (1 + 1e-12)][0]
    assert (F.info["rule_log2s"], F.info["rule_ratio"]) == first


def test_fallback_reverts_to_uniform_placement():
    """Appendix E's fallback: with the threshold at 0 every non-uniform choice
    falls back, and then the codebooks are the uniform placement over the
    initial pairs and every group re-picks by Eq. (5); the two- and six-bit
    errors that decided it match a recomputation through the quantizer (the
    plane rule carried to six bits)."""
    w, _ = synth_matrix(4, 128, "student_t", 9)
    E = synth_channel_energy(128, 9)
    g, N = 32, 4
    F0 = oracle.encode_full(w, g, N, E=E, fallback=np.inf)
    F = oracle.encode_full(w, g, N, E=E, fallback=0.0)
    if (F0.info["rule_log2s"], F0.info["rule_ratio"]) == ("uniform", "uniform"):
        pytest.skip("the best rule pair is already uniform")
    assert F.info["fell_back"] and F.info["rule_log2s"] == F.info["rule_ratio"] == "uniform"
    pre = _ratio_pre_grid(w, g, 4.0).reshape(4, 4, g)
    lo64 = np.where(pre, np.inf, w.astype(np.float64).reshape(4, 4, g)).min(axis=2)
    hi64 = np.where(pre, -np.inf, w.astype(np.float64).reshape(4, 4, g)).max(axis=2)
    lo0, s0 = oracle.initial_pair(lo64, hi64)
    cs, cr = oracle.uniform_codebooks(lo0, s0)
    assert np.array_equal(F.cb_log2s.view(np.uint16), cs.view(np.uint16))
    assert np.array_equal(F.cb_ratio.view(np.uint16), cr.view(np.uint16))
    # the errors of the pre-fallback choice, through the quantizer
    tlo, ts = oracle.codebook_table(F0.cb_log2s, F0.cb_ratio)
    e2 = e6 = 0.0
    v = np.clip(w.astype(np.float64).reshape(4, 4, g), lo64[..., None], hi64[..., None])
    for r in range(4):
        for gi in range(4):
            lo, s = float(tlo[F0.idx[r, gi]]), float(ts[F0.idx[r, gi]])
            for j in range(g):
                x, e = float(v[r, gi, j]), E[gi * g + j]
                q, b = oracle.quantize_value(x, lo, s, 6)
                rec = lo + s * q
                e2 += e * (x - rec) ** 2
                for k in range(3, 7):
                    rec += (2 * b[k - 3] - 1) * s / 2.0 ** (k - 1)
                e6 += e * (x - rec) ** 2
    assert math.isclose(F.info["err2"], e2, rel_tol=1e-12)
    assert math.isclose(F.info["err6"], e6, rel_tol=1e-12)
    # at the paper's threshold the decision is the comparison of these two
    Fd = oracle.encode_full(w, g, N, E=E)
    assert Fd.info["fell_back"] == (e6 > 0.1 * e2)


# ------------------------------------------------------- guards (Eq. 11)
def test_entry_bits_closed_form():
    """Appendix E's charge: 8 code bits + log2(n/k) + log2 e per pre-grid
    entry; 16 + ceil(log2 C) per post-grid entry."""
    assert math.isclose(oracle.entry_bits(1024, 4), 8 + 8 + 1 / math.log(2), rel_tol=1e-15)
    assert math.isclose(oracle.entry_bits(4096, 4096), 8 + 1 / math.log(2), rel_tol=1e-15)
    assert oracle.post_bits(4096) == 28 and oracle.post_bits(4097) == 29 and oracle.post_bits(1000) == 26


def test_clip_candidate_moves_the_extreme_to_the_next_value_inward():
    j, v = oracle.clip_candidate(np.array([0.1, -0.9, 0.3, -0.2]))
    assert j == 1 and list(v) == [0.1, -0.2, 0.3, -0.2]
    j, v = oracle.clip_candidate(np.array([0.1, 0.9, 0.3, -0.2]))
    assert j == 1 and list(v) == [0.1, 0.3, 0.3, -0.2]
    j, v = oracle.clip_candidate(np.array([0.5, -0.5, 0.0]))   # tie: lowest column, the maximum
    assert j == 0 and list(v) == [0.0, -0.5, 0.0]


def _best_pair_exact(vals, wts, tlo, ts, N, lam):
    losses = [_exact_loss(vals, wts, float(tlo[c]), float(ts[c]), N, lam) for c in range(256)]
    return losses.index(min(losses))


def _d2_via_quantizer(vals, wts, lo, s):
    tot = 0.0
    for v, e in zip(vals, wts):
        q, _ = oracle.quantize_value(v, lo, s, 2)
        tot += e * (v - (lo + s * q)) ** 2
    return tot


def test_gain_is_the_fall_in_two_bit_error_after_the_refit():
    """Eq. (11) with reading FE5, group by group: the pair re-picked by Eq. (5)
    (checked in exact rationals) for the group as is and with its candidate
    clipped, and the two-bit errors recomputed through the single-value
    quantizer; the held-out set is exactly the gains per bit above tau."""
    w, _ = synth_matrix(2, 32, "student_t", 12)
    w[1, 20] = np.float16(0.5)
    E = synth_channel_energy(32, 12)
    g, N, tau = 16, 3, 1e-6
    F = oracle.encode_full(w, g, N, E=E, criterion="gain", tau=tau)
    gain = F.info["gain"]
    wg = w.astype(np.float64).reshape(2, 2, g)
    lo0, s0 = oracle.initial_pair(wg.min(axis=2), wg.max(axis=2))
    tlo, ts = oracle.codebook_table(*oracle.uniform_codebooks(lo0, s0))
    for r in range(2):
        for gi in range(2):
            vals = [float(v) for v in wg[r, gi]]
            wts = E[gi * g:(gi + 1) * g]
            j = max(range(g), key=lambda i: (abs(vals[i]), -i))
            others = vals[:j] + vals[j + 1:]
            clipped = list(vals)
            clipped[j] = max(others) if vals[j] >= max(others) else min(others)
            c0 = _best_pair_exact(vals, wts, tlo, ts, N, 4)
            c1 = _best_pair_exact(clipped, wts, tlo, ts, N, 4)
            want = _d2_via_quantizer(vals, wts, float(tlo[c0]), float(ts[c0])) - \
                _d2_via_quantizer(clipped, wts, float(tlo[c1]), float(ts[c1]))
            assert math.isclose(gain[r, gi], want, rel_tol=1e-9, abs_tol=1e-18)
    k = F.n_pre
    assert k == int((gain / oracle.entry_bits(w.size, max(k, 1)) > tau).sum())
    assert F.mask[1, 20]


def test_gain_threshold_is_monotone():
    """tau = 0 holds out every candidate with a positive gain; a larger tau
    never holds out more; an infinite tau holds out nothing (and keeps no
    post-grid entry either)."""
    w, _ = synth_matrix(8, 128, "student_t", 13)
    E = synth_channel_energy(128, 13)
    counts = []
    for tau in (0.0, 1e-6, 1e-5, 1e-4, np.inf):
        F = oracle.encode_full(w, 32, 4, E=E, criterion="gain", tau=tau)
        counts.append((F.n_pre, F.n_post))
        if tau == 0.0:
            assert F.n_pre == int((F.info["gain"] > 0).sum())
    assert all(a[0] >= b[0] and a[1] >= b[1] for a, b in zip(counts, counts[1:]))
    assert counts[-1] == (0, 0)


def _ratio_pre_grid(w, g, T):
    """The ratio criterion written out per group (section 3.5)."""
    R, C = w.shape
    pre = np.zeros((R, C), bool)
    for r in range(R):
        for gi in range(C // g):
            seg = [abs(float(x)) for x in w[r, gi * g:(gi + 1) * g]]
            j = seg.index(max(seg))
            second = max(seg[:j] + seg[j + 1:])
            if seg[j] > T * second:
                pre[r, gi * g + j] = True
    return pre


@pytest.mark.parametrize("criterion", ["ratio", "gain"])
def test_post_grid_picks_per_row_by_brute_force(criterion):
    """Appendix E's post-grid guard, row by row in plain Python: under the
    ratio criterion the one entry with the largest E_c-weighted two-bit error
    (lowest column on ties) among those the pre-grid guard left; under the gain
    criterion the three best such errors per stored bit, kept above tau."""
    w, _ = synth_matrix(6, 128, "normal_outliers", 14)
    E = synth_channel_energy(128, 14)
    g, N, tau = 32, 4, 2e-6
    F = oracle.encode_full(w, g, N, E=E, criterion=criterion, tau=tau)
    if criterion == "ratio":
        pre = _ratio_pre_grid(w, g, 4.0)
    else:
        hold = F.info["gain"] / oracle.entry_bits(w.size, max(F.n_pre, 1)) > tau
        pre = np.zeros_like(F.mask)
        for r in range(F.rows):
            for gi in range(F.cols // g):
                if hold[r, gi]:
                    seg = [abs(float(x)) for x in w[r, gi * g:(gi + 1) * g]]
                    pre[r, gi * g + seg.index(max(seg))] = True
    assert int(pre.sum()) == F.n_pre
    for r in range(F.rows):
        errs = []
        for c in range(F.cols):
            if pre[r, c]:
                continue
            lo, s = float(F.lo[r, c // g]), float(F.s[r, c // g])
            q = 0 if s == 0 else sum(1 for j in range(3) if float(w[r, c]) - lo >= (j + 0.5) * s)
            errs.append((E[c] * (float(w[r, c]) - (lo + s * q)) ** 2, c))
        errs.sort(key=lambda t: (-t[0], t[1]))
        if criterion == "ratio":
            want = {errs[0][1]}
        else:
            want = {c for e, c in errs[:3] if e / oracle.post_bits(F.cols) > tau}
        got = set(np.nonzero(F.mask[r] & ~pre[r])[0].tolist())
        assert got == want, r


# ------------------------------------------------------------ invariants
@pytest.mark.parametrize("criterion", ["ratio", "gain"])
def test_full_encoder_invariants(criterion):
    """Whatever the guards chose: held-out entries decode to the weight itself
    at every precision (Eq. 4), their planes are zero, codes keep the prefix
    property, the pairs are the table entries the indices select, and every
    main-stream entry is within t_M of its clipped value or beyond the grid's
    reach only by what clipping removed."""
    w, _ = synth_matrix(16, 256, "student_t", 15)
    E = synth_channel_energy(256, 15)
    F = oracle.encode_full(w, 64, 5, E=E, criterion=criterion, tau=1e-5)
    tlo, ts = oracle.codebook_table(F.cb_log2s, F.cb_ratio)
    assert np.array_equal(F.s.view(np.uint16), ts[F.idx].view(np.uint16))
    for M in range(2, 6):
        wh = oracle.w_hat(F, M)
        assert np.array_equal(wh[F.mask], w.astype(np.float64)[F.mask])
        if M < 5:
            assert np.array_equal(oracle.codes(F, M), oracle.codes(F, 5) >> (5 - M))
    assert not F.planes[:, F.mask].any()
    assert F.row_ptr[-1] == F.nnz == int(F.mask.sum()) == F.n_pre + F.n_post


def test_fitted_grids_sit_off_the_group_extremes():
    """Section 3.1: under the Eq. (5) choice no level sits on a group extreme;
    the min-max fit puts the lowest level on every group's minimum."""
    w, _ = synth_matrix(32, 512, "student_t", 16)
    F = oracle.encode_full(w, 128, 4, E=synth_channel_energy(512, 16))
    wg = w.astype(np.float64).reshape(32, 4, 128)
    lo, s = F.lo.astype(np.float64), F.s.astype(np.float64)
    assert np.mean(lo == wg.min(axis=2)) < 0.05 and np.mean(lo + 3 * s == wg.max(axis=2)) < 0.05
    F0 = oracle.encode(w, 128, 4, 0.0)
    assert np.all(F0.lo.astype(np.float64) == wg.min(axis=2))


def test_channel_energy_recipe():
    """The synthetic E_c: positive, seeded, round(0.005 C) channels (at least
    one) lifted by 100 above a log-normal body."""
    e = synth_channel_energy(4096, 3)
    assert e.shape == (4096,) and np.all(e > 0) and np.array_equal(e, synth_channel_energy(4096, 3))
    # 20 lifted channels sit near ln 100 = 4.6 in log space, the body near 0:
    # about 17 of the 20 and 1 of the body lie above 3.5
    assert 10 <= int((np.log(e) > 3.5).sum()) <= 25


@pytest.mark.parametrize("criterion", ["ratio", "gain"])
def test_paper_side_record_codes(criterion):
    """Appendix E's side-record codes (reading FE8), entry by entry in plain
    Python: post-grid entries hold the two-bit base plus the fp16 residual;
    pre-grid entries hold w in fp16 under the ratio criterion, and under the
    gain criterion an 8-bit code times the row's fp16 scale (the largest |w| of
    the row's pre-grid entries / 127), within half a scale step of w; every
    value is rounded once to fp16.  Nothing but the recorded values changes."""
    w, x = synth_matrix(12, 256, "normal_outliers", 23)
    E = synth_channel_energy(256, 23)
    Fw = oracle.encode_full(w, 64, 4, E=E, criterion=criterion, tau=1e-5)
    F = oracle.encode_full(w, 64, 4, E=E, criterion=criterion, tau=1e-5, storage="paper")
    for k in ("q", "planes", "mask", "row_ptr", "col", "idx"):
        assert np.array_equal(getattr(F, k), getattr(Fw, k)), k
    assert np.array_equal(Fw.val, w[Fw.mask])          # storage "weight": w itself
    if criterion == "ratio":
        pre = _ratio_pre_grid(w, 64, 4.0)
    else:
        hold = F.info["gain"] / oracle.entry_bits(w.size, max(F.n_pre, 1)) > 1e-5
        pre = np.zeros_like(F.mask)
        for r in range(12):
            for gi in range(4):
                if hold[r, gi]:
                    seg = [abs(float(v)) for v in w[r, gi * 64:(gi + 1) * 64]]
                    pre[r, gi * 64 + seg.index(max(seg))] = True
    n_checked = {"pre": 0, "post": 0}
    for r in range(12):
        pre_cols = [c for c in range(256) if pre[r, c]]
        scale = float(np.float16(max(abs(float(w[r, c])) for c in pre_cols) / 127)) if pre_cols else 0.0
        for e in range(F.row_ptr[r], F.row_ptr[r + 1]):
            c = int(F.col[e])
            wv = float(w[r, c])
            got = float(F.val[e])
            if pre[r, c]:
                if criterion == "ratio":
                    want = wv
                else:
                    code = max(-127, min(127, round(wv / scale)))   # Python round: half to even
                    want = float(np.float16(code * scale))
                    assert abs(code * scale - wv) <= scale / 2 + 1e-12
                n_checked["pre"] += 1
            else:
                lo, s = float(F.lo[r, c // 64]), float(F.s[r, c // 64])
                base = lo + s * int(F.q[r, c])
                want = float(np.float16(base + float(np.float16(wv - base))))
                n_checked["post"] += 1
            assert got == want, (r, c)
    assert n_checked["pre"] > 0 and n_checked["post"] > 0
    y = oracle.gemv(F, x, 3)                               # the recorded values are what W_hat uses
    assert np.allclose(oracle.w_hat(F, 3)[F.mask], F.val.astype(np.float64))
    assert np.isfinite(y).all()
