"""The full StagQ encoder: codebook placement rules, the activation-weighted
pair choice, the gain criterion and the per-row post-grid guard.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the CPU-baseline leg of the benchmark may import it, and it
shares no code with the HIP library.  It produces a second, differently shaped
workload for the GEMV's parity tests (grids whose levels sit off the group
extremes, per-row side records); the GEMV consumes its fields like any other.

It follows the StagQ paper ("StagQ: Constraint-Driven Multi-Precision Weight
Quantization for LLMs"): section 3.1 with Eq. (5) and Eq. (6) for the pair,
section 3.5 with Eq. (11) for the gain criterion, section 3.6 and Figure 3 for
the order of the stages (pre-grid guard -> pair fit -> base code -> post-grid
guard -> planes), and Appendix E ("Base" and "Guards") for the placement
rules, the rule choice, the fallback and the post-grid picks.  The AWQ scale of
section 3.6 is outside: the input is already the scaled matrix, and E holds
the calibration mean square of each input channel.

Readings (where the paper is silent or leaves a choice open)
------------------------------------------------------------
FE1  E_c is given per input channel (the tests draw a synthetic, seeded one);
    E = None means E_c = 1.  Every error below is weighted by E_c, as Eq. (5)
    and Eq. (6) weight theirs.
FE2  The codebooks are placed over log2 s0 and lo0 / s0 of the initial pairs
    (Appendix B) of the groups with s0 > 0, the pre-grid entries clipped.
    Lloyd's rule is the unweighted one-dimensional k-means with 16 centres,
    started from the uniform placement; a value goes to its nearest centre (the
    lower one on ties), a centre moves to the mean of its values (an empty cell
    keeps its centre), and it stops when no centre moves (at most 200 rounds).
    The anchored rule keeps the first and last centres at the ends of the range.
FE3  The rule pair is chosen by the first term of Eq. (5) summed over the
    matrix, each group taking its best pair under that term alone; the nine
    combinations are tried with the log2 s rule outer, in the order uniform,
    Lloyd, anchored Lloyd, and a later one must be strictly better to win.
FE4  The fallback compares errors summed over the matrix (E_c-weighted, final
    per-group choice): the "six-bit error" is that of the six-bit prefix
    reconstruction, the plane rule carried to plane 6 even where fewer planes
    are stored; above a tenth of the two-bit error, both codebooks revert to
    uniform placement and every group picks again.
FE5  Gain criterion: a group's candidate is its largest-|w| entry (lowest column
    on ties), clipped to the nearest other value of the group toward the inside
    (the largest of the others if it is the group maximum, else the smallest).
    Scoring re-picks that group's pair among the 256 of codebooks placed
    uniformly over the unclipped initial pairs; the codebooks are not refitted
    per candidate.  D2(V) = sum_c E_c (v_c - (lo + s q_c))^2 over the values of
    its argument, with the pair the Eq. (5) choice makes for them.
FE6  The bits a pre-grid entry occupies are b = 8 + log2(n / k) + log2 e
    (Appendix E's 8-bit code and position charge, n weights, k held out), with
    k solved by a fixed-point iteration that starts from the number of
    positive gains (k can only fall, so it settles).
FE7  Post-grid guard over the entries the pre-grid guard left: under the ratio
    criterion exactly one entry per row, the largest E_c (w - (lo + s q))^2
    (lowest column on ties); under the gain criterion that error per stored
    bit, b_post = 16 + ceil(log2 C) (an fp16 residual and a column index), the
    three highest of each row kept when above tau.
FE8  storage "weight": the side record stores the held-out weight itself as
    fp16 (reading R6 of the main oracle module).  storage "paper": the side-
    record codes of Appendix E -- a pre-grid entry of the gain criterion is an
    8-bit symmetric code against one fp16 scale per row (scale = fp16(largest
    |w| of the row's pre-grid entries / 127), code = w / scale rounded to
    nearest even and clamped to [-127, 127], value code * scale); a pre-grid
    entry of the ratio criterion is w in fp16; a post-grid entry is its fp16
    residual against the two-bit base (value lo + s q + fp16(w - (lo + s q))).
    The record the GEMV reads holds one fp16 value per entry, so each value is
    rounded once to fp16.  Neither guard has a budget cap.

Pinned by tests/test_oracle_full_encoder.py: Lloyd fixed points and monotone
distortion, the rule choice and fallback against brute force through the
decoder, the weighted choice against an exact-rational loss, the gain against
two-bit errors recomputed through the decoder, the per-row picks by brute
force, and the encoder invariants.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

from .stagq_oracle import Fields, codebook_table, initial_pair, pair_loss, uniform_codebooks

__all__ = ["lloyd_1d", "place_codebook", "pick_pairs", "two_bit_error", "clip_candidate",
           "entry_bits", "post_bits", "encode_full", "RULES"]

RULES = ("uniform", "lloyd", "lloyd_anchored")


def lloyd_1d(values, init, anchored: bool = False, max_iter: int = 200) -> np.ndarray:
    """Lloyd's rule on the real line (reading FE2): alternate nearest-centre
    assignment (lower centre on ties) and centre = mean of its cell; anchored
    keeps the first and last centres where init put them."""
    v = np.asarray(values, dtype=np.float64).ravel()
    c = np.asarray(init, dtype=np.float64).copy()
    for _ in range(max_iter):
        cell = np.argmin(np.abs(v[:, None] - c[None, :]), axis=1)   # first minimum = lower centre
        new = c.copy()
        for k in range(c.shape[0]):
            if anchored and (k == 0 or k == c.shape[0] - 1):
                continue
            sel = v[cell == k]
            if sel.size:
                new[k] = sel.mean()
        if np.array_equal(new, c):
            break
        c = new
    return c


def place_codebook(values, rule: str) -> np.ndarray:
    """One 16-entry fp16 codebook over values by rule (Appendix E "Base")."""
    v = np.asarray(values, dtype=np.float64).ravel()
    init = v.min() + np.arange(16, dtype=np.float64) / 15.0 * (v.max() - v.min())
    if rule == "uniform":
        c = init
    elif rule == "lloyd":
        c = lloyd_1d(v, init)
    elif rule == "lloyd_anchored":
        c = lloyd_1d(v, init, anchored=True)
    else:
        raise ValueError(f"unknown placement rule {rule!r}")
    return c.astype(np.float16)


def pick_pairs(v, E, tlo, ts, nbits: int, lam: float) -> Tuple[np.ndarray, np.ndarray]:
    """Per group (last axis of v) the index among the 256 pairs minimizing
    Eq. (5) with floor weight lam (lowest index on ties); returns (idx, loss)."""
    best = np.full(v.shape[:-1], np.inf)
    idx = np.zeros(v.shape[:-1], dtype=np.uint8)
    for c in range(256):
        D = pair_loss(v, np.full(v.shape[:-1], float(tlo[c])), np.full(v.shape[:-1], float(ts[c])),
                      nbits, lam, E=E)
        better = D < best
        best = np.where(better, D, best)
        idx = np.where(better, np.uint8(c), idx)
    return idx, best


def _base_code(v, lo, s):
    """Nearest of lo + j s (ties up), j = 0..3; 0 where s = 0."""
    q = np.zeros(v.shape, dtype=np.float64)
    for j in range(3):
        q += (v - lo >= (j + 0.5) * s)
    return np.where(s > 0.0, q, 0.0)


def two_bit_error(v, E, lo, s) -> np.ndarray:
    """D2 = sum_c E_c (v_c - (lo + s q_c))^2 over the last axis (reading FE5)."""
    v = np.asarray(v, dtype=np.float64)
    wt = np.broadcast_to(np.asarray(E, dtype=np.float64), v.shape)
    lo = np.asarray(lo, dtype=np.float64)[..., None]
    s = np.asarray(s, dtype=np.float64)[..., None]
    return (wt * (v - (lo + s * _base_code(v, lo, s))) ** 2).sum(axis=-1)


def _prefix_error(v, E, lo, s, M: int) -> float:
    """sum E_c (v - W^(M))^2 with the plane rule carried to plane M (FE4)."""
    lo = lo[..., None]
    s = s[..., None]
    rec = lo + s * _base_code(v, lo, s)
    for k in range(3, M + 1):
        b = (v - rec) >= 0.0
        rec = rec + np.where(s > 0.0, (2.0 * b - 1.0) * s / 2.0 ** (k - 1), 0.0)
    return float((E * (v - rec) ** 2).sum())


def clip_candidate(g: np.ndarray) -> Tuple[int, np.ndarray]:
    """The gain criterion's candidate in one group (reading FE5): its position
    and the group's values with it clipped to the next value inward."""
    g = np.asarray(g, dtype=np.float64)
    j = int(np.argmax(np.abs(g)))
    others = np.delete(g, j)
    out = g.copy()
    if others.size:
        out[j] = others.max() if g[j] >= others.max() else others.min()
    return j, out


def entry_bits(n: int, k: int) -> float:
    """Bits of one pre-grid entry under the gain criterion (FE6)."""
    return 8.0 + math.log2(n / k) + math.log2(math.e)


def post_bits(cols: int) -> float:
    """Bits of one post-grid entry under the gain criterion (FE7)."""
    return 16.0 + math.ceil(math.log2(cols))


def _fit_pairs(v, E, nbits, lam, lo64, hi64, fallback):
    """Codebooks by the best of the nine rule pairs (FE2, FE3), the per-group
    choice by Eq. (5), and the fallback (FE4)."""
    lo0, s0 = initial_pair(lo64, hi64)
    pos = s0 > 0.0
    if pos.any():
        L = np.log2(s0[pos])
        P = lo0[pos] / s0[pos]
    else:
        L = P = np.zeros(1)
    best = None
    for rs in RULES:
        cs = place_codebook(L, rs)
        for rr in RULES:
            cr = place_codebook(P, rr)
            tlo, ts = codebook_table(cs, cr)
            _, first = pick_pairs(v, E, tlo, ts, nbits, 0.0)
            score = float(first.sum())
            if best is None or score < best[0]:
                best = (score, rs, rr, cs, cr)
    _, rs, rr, cs, cr = best
    tlo, ts = codebook_table(cs, cr)
    idx, _ = pick_pairs(v, E, tlo, ts, nbits, lam)
    e2 = _prefix_error(v, E, tlo[idx].astype(np.float64), ts[idx].astype(np.float64), 2)
    e6 = _prefix_error(v, E, tlo[idx].astype(np.float64), ts[idx].astype(np.float64), 6)
    fell_back = e6 > fallback * e2 and (rs, rr) != ("uniform", "uniform")
    if fell_back:
        rs = rr = "uniform"
        cs, cr = uniform_codebooks(lo0, s0)
        tlo, ts = codebook_table(cs, cr)
        idx, _ = pick_pairs(v, E, tlo, ts, nbits, lam)
    return idx, cs, cr, tlo, ts, dict(rule_log2s=rs, rule_ratio=rr, fell_back=bool(fell_back),
                                      err2=e2, err6=e6)


def encode_full(w16: np.ndarray, group: int, nbits: int, E: Optional[np.ndarray] = None,
                criterion: str = "ratio", T: float = 4.0, tau: float = 1e-8,
                lam: float = 4.0, fallback: float = 0.1, storage: str = "weight") -> Fields:
    """The full encoder in Figure 3's order.  criterion "ratio": the pre-grid
    guard of section 3.5 with factor T and one post-grid entry per row;
    "gain": Eq. (11) with threshold tau for both guards.  The pair is always
    the codebook metadata of section 3.1; fallback is the ratio of six-bit to
    two-bit error above which the codebooks revert to uniform placement (a
    tenth in Appendix E); storage selects how the side record holds its
    values (FE8).  Returns Fields with .info."""
    if criterion not in ("ratio", "gain"):
        raise ValueError("criterion must be 'ratio' or 'gain'")
    if storage not in ("weight", "paper"):
        raise ValueError("storage must be 'weight' or 'paper'")
    w16 = np.asarray(w16)
    if w16.ndim != 2 or w16.dtype != np.float16:
        raise ValueError("encode_full expects a 2-D float16 matrix")
    R, C = w16.shape
    if C % group != 0 or nbits < 2:
        raise ValueError("cols must be a multiple of the group size and nbits >= 2")
    G = C // group
    Ec = np.ones(C) if E is None else np.asarray(E, dtype=np.float64)
    if Ec.shape != (C,) or not np.all(np.isfinite(Ec)) or np.any(Ec <= 0.0):
        raise ValueError("E must hold one positive mean square per input channel")
    Eg = np.broadcast_to(Ec.reshape(1, G, group), (R, G, group))
    w = w16.astype(np.float64)
    wg = w.reshape(R, G, group)
    mask = np.zeros((R, G, group), dtype=bool)
    info = dict(criterion=criterion)

    # 1. Pre-grid guard (section 3.5).
    if criterion == "ratio":
        mag = np.abs(wg)
        i_max = np.argmax(mag, axis=2)
        a = np.take_along_axis(mag, i_max[..., None], axis=2)[..., 0]
        others = mag.copy()
        np.put_along_axis(others, i_max[..., None], -1.0, axis=2)
        hold = a > T * others.max(axis=2)
        rr, gg = np.nonzero(hold)
        mask[rr, gg, i_max[rr, gg]] = True
    elif group > 1:
        # Eq. (11): gain of clipping each group's candidate, per bit of storage
        lo0, s0 = initial_pair(wg.min(axis=2), wg.max(axis=2))
        cs, cr = uniform_codebooks(lo0, s0)
        tlo, ts = codebook_table(cs, cr)
        jj = np.zeros((R, G), dtype=np.int64)
        vc = wg.copy()
        for r in range(R):
            for gi in range(G):
                jj[r, gi], vc[r, gi] = clip_candidate(wg[r, gi])
        i0, _ = pick_pairs(wg, Eg, tlo, ts, nbits, lam)
        i1, _ = pick_pairs(vc, Eg, tlo, ts, nbits, lam)
        d_before = two_bit_error(wg, Eg, tlo[i0].astype(np.float64), ts[i0].astype(np.float64))
        d_after = two_bit_error(vc, Eg, tlo[i1].astype(np.float64), ts[i1].astype(np.float64))
        gain = d_before - d_after
        k = int((gain > 0.0).sum())
        while k > 0:
            k_new = int((gain / entry_bits(R * C, k) > tau).sum())
            if k_new == k:
                break
            k = k_new
        if k > 0:
            hold = gain / entry_bits(R * C, k) > tau
            rr, gg = np.nonzero(hold)
            mask[rr, gg, jj[rr, gg]] = True
        info["gain"] = gain
    n_pre = int(mask.sum())
    pre_mask = mask.reshape(R, C).copy()

    # 2. Pair fit over the group with its pre-grid entry clipped to the next
    #    value inward (= clamped to the range of the others), section 3.1.
    lo64 = np.where(mask, np.inf, wg).min(axis=2)
    hi64 = np.where(mask, -np.inf, wg).max(axis=2)
    v = np.clip(wg, lo64[..., None], hi64[..., None])
    idx, cb_log2s, cb_ratio, tlo, ts, fit = _fit_pairs(v, Eg, nbits, lam, lo64, hi64, fallback)
    info.update(fit)
    lo16, s16 = tlo[idx], ts[idx]
    lo_f = lo16.astype(np.float64)[..., None]
    s_f = s16.astype(np.float64)[..., None]

    # 3. Base code of every entry from its original value (ties up).
    q = _base_code(wg, lo_f, s_f).astype(np.int64)

    # 4. Post-grid guard, per output row (Appendix E "Guards", reading FE7).
    err2 = (Eg * (wg - (lo_f + s_f * q)) ** 2).reshape(R, C)
    free = ~mask.reshape(R, C)
    post = np.zeros((R, C), dtype=bool)
    for r in range(R):
        cols = np.nonzero(free[r])[0]
        if cols.size == 0:
            continue
        e = err2[r, cols]
        order = np.lexsort((cols, -e))              # error descending, then column
        if criterion == "ratio":
            post[r, cols[order[0]]] = True
        else:
            top = order[:3]
            keep = e[top] / post_bits(C) > tau
            post[r, cols[top[keep]]] = True
    mask |= post.reshape(R, G, group)
    n_post = int(post.sum())

    # 5. Planes: sign of the prefix residual; skipped at held-out positions and
    #    in zero-step groups.
    planes = np.zeros((nbits - 2, R, G, group), dtype=np.uint8)
    rec = lo_f + s_f * q
    active = (~mask) & (s_f > 0.0)
    for k in range(3, nbits + 1):
        bk = ((wg - rec) >= 0.0) & active
        planes[k - 3] = bk
        rec = rec + np.where(active, (2.0 * bk - 1.0) * s_f / 2.0 ** (k - 1), 0.0)

    # 6. Side record, CSR by (row, col): the held-out weight itself, or the
    #    paper's codes (FE8).
    mask2 = mask.reshape(R, C)
    rr, cc = np.nonzero(mask2)
    P = w.copy()
    if storage == "paper":
        base = (lo_f + s_f * q).reshape(R, C)                  # exact
        r16 = (w - base).astype(np.float16).astype(np.float64)  # fp16 residual
        P = np.where(post, base + r16, P)
        if criterion == "gain":
            for r in range(R):
                cols = np.nonzero(pre_mask[r])[0]
                if cols.size == 0:
                    continue
                scale = float(np.float16(np.abs(w[r, cols]).max() / 127.0))
                code = np.clip(np.rint(w[r, cols] / scale), -127, 127) if scale > 0 else 0.0 * cols
                P[r, cols] = code * scale
    val = P[rr, cc].astype(np.float16)
    row_ptr = np.zeros(R + 1, dtype=np.int64)
    np.add.at(row_ptr, rr + 1, 1)
    row_ptr = np.cumsum(row_ptr).astype(np.int32)
    return Fields(
        rows=R, cols=C, group=group, nbits=nbits,
        q=q.reshape(R, C).astype(np.uint8), planes=planes.reshape(nbits - 2, R, C),
        lo=lo16, s=s16, mask=mask2, row_ptr=row_ptr, col=cc.astype(np.int32),
        val=val, n_pre=n_pre, n_post=n_post,
        idx=idx, cb_log2s=cb_log2s, cb_ratio=cb_ratio, info=info)
