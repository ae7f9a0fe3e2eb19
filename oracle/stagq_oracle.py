"""Plain CPU oracle for the StagQ batch-one GEMV.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the product path (the HIP library
and its Python binding) never does.  It shares no code with the product: every
step below is written from the StagQ paper ("StagQ: Constraint-Driven
Multi-Precision Weight Quantization for LLMs"), in float64 NumPy, slowly and
in the paper's order, so that a reader can check it against the text by eye.

What is computed
----------------
encode()      the reference encoder.  The paper's encoder (section 3.6,
              Figure 3, Appendix E) runs pre-grid guard -> pair fit -> base
              code -> post-grid guard -> planes.  Calibration data are not
              available, so the activation scale is omitted and every weight
              counts equally (E_c = 1); the pair is the conventional min-max
              lattice of section 3.1 / Appendix D; the pre-grid guard is the
              ratio criterion of section 3.5.  Options: the codebook
              metadata of section 3.1 (pair_fit="codebook") and per-row
              post-grid picks (post_per_row).  The full encoder, with
              calibration weights, Lloyd placement and the gain criterion,
              is in stagq_encoder_full.py.
codes()       the composite integer u_M of Eq. (8).
w_main()      the additive reconstruction of Eq. (9) (the direct form; the GPU
              path uses the affine collapse of Eq. (10) instead).
w_hat()       the complete reconstruction of Eq. (4): main stream outside the
              side record, the recorded value inside it.
gemv()        y = W_hat^(M) x in float64.
scale_x()     the activation a decoder feeds the GEMV when it applies the
              inverse AWQ scale at run time (section 3.6, Appendix E: the
              quantizer works on W diag(a), so x is divided by a per input
              channel), and gemv_scaled() = gemv(scale_x(x)).

Readings of the paper (where it is silent or leaves a choice open)
------------------------------------------------------------------
R1  "Nearest rounding" of the base code breaks ties upward, the same way the
    planes treat a zero residual (sign(0) := +1, section 3.3).
R2  The pair is fitted to the non-held-out entries of the group: lo = min,
    s = (max - min)/3, so the outer two base levels sit on the group extremes
    (the conventional four-level lattice of section 3.1).  This equals the
    paper's "held-out entry clipped to the next value inward".  The pair is
    stored as two fp16 numbers; every later step uses the stored values.
R3  Pre-grid guard = ratio criterion with T = 4 (section 3.5, Table 6): in
    each group, the largest |w| (lowest column on ties) is a candidate when it
    exceeds T times the second largest.  Candidates are ranked by that ratio
    (infinite when the second largest is 0; ties by flat index) and the first
    min(K, #candidates) are held out, K = round(frac * R * C).
R4  Post-grid guard: the remaining budget K - K_pre goes to the entries with
    the largest two-bit residual |w - (lo + s q)| over the whole matrix (ties
    by flat index).  The paper picks per output row with activation weights
    (Appendix E); encode(..., post_per_row=k) takes the k largest residuals of
    every row instead (ties by column, every channel weighing the same; K then
    caps the pre-grid guard only).  The full encoder in stagq_encoder_full.py
    has the activation-weighted per-row pick.
R5  Held-out entries keep the base code of their original value and all-zero
    planes: the planes "skip every position the side record already carries"
    (section 3.6), and Eq. (4)'s (1 - m) removes whatever the main stream
    decodes there.
R6  The side record stores the held-out weight itself as fp16.  For fp16
    weights this equals both of the paper's definitions of P (section 3).
R7  A group whose stored step is 0 gets q = 0 and all-zero planes.
R8  The run-time inverse scale arrives as one fp16 factor per input channel
    (1 / a_c), and the scaled activation is the fp16 rounding (nearest, ties to
    even) of the exact product x_c * (1 / a_c): the GEMV's activations are fp16.
R9  Codebook metadata: the initial pair (Appendix B) puts the outer two of four
    symmetric levels 6% of the group range in from either end, so its step is
    0.88 / 3 = 0.2933 of the range (the page's "0.29").
R10 The 256 (lo, s) pairs are s = fp16(2^c_s[i]) and lo = fp16(c_r[j] * s) from
    the fp16 codebook entries, and index i * 16 + j is the stored byte.  Of the
    page's three placement rules encode(..., pair_fit="codebook") uses only
    uniform placement (its fallback); stagq_encoder_full.py has all three.
R11 In the per-group loss, the pre-grid entry "clipped to the next value
    inward" is clamped to the range of the group's other entries; E_c = 1 in
    encode() (stagq_encoder_full.py takes E_c); lambda = 4; the lowest index
    wins ties.

Parity status of every function is recorded next to it ("pinned by ...").
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Fields", "encode", "quantize_value", "codes", "w_main", "w_hat", "gemv",
    "half_step", "affine_pair", "budget", "scale_x", "gemv_scaled",
    "initial_pair", "uniform_codebooks", "codebook_table", "pair_loss",
]


@dataclass
class Fields:
    """Unpacked encoder output (the fields the main stream and side record hold)."""
    rows: int
    cols: int
    group: int
    nbits: int                 # N: q plus planes k = 3..N
    q: np.ndarray              # uint8 [R, C], 0..3
    planes: np.ndarray         # uint8 [N-2, R, C], 0/1, plane k = 3 first
    lo: np.ndarray             # float16 [R, G]
    s: np.ndarray              # float16 [R, G]
    mask: np.ndarray           # bool [R, C], held-out entries (m of Eq. 4)
    row_ptr: np.ndarray        # int32 [R + 1]
    col: np.ndarray            # int32 [nnz]
    val: np.ndarray            # float16 [nnz], the recorded value P
    n_pre: int = 0             # entries held out by the pre-grid guard
    n_post: int = 0            # entries held out by the post-grid guard
    # codebook metadata (encode(..., pair_fit="codebook") only): per group an
    # 8-bit index i * 16 + j into two 16-entry fp16 codebooks, log2 s and lo/s
    idx: Optional[np.ndarray] = None       # uint8 [R, G]
    cb_log2s: Optional[np.ndarray] = None  # float16 [16]
    cb_ratio: Optional[np.ndarray] = None  # float16 [16]
    # what the full encoder chose (codebook rules, guard counts), if it ran
    info: Optional[dict] = None

    @property
    def nnz(self) -> int:
        return int(self.col.shape[0])

    def as_dict(self) -> Dict[str, np.ndarray]:
        return dict(q=self.q, planes=self.planes, lo=self.lo, s=self.s, mask=self.mask,
                    row_ptr=self.row_ptr, col=self.col, val=self.val)


def budget(frac: float, rows: int, cols: int) -> int:
    """Side-record size K = round(frac * R * C), halves rounded up."""
    return int(np.floor(frac * rows * cols + 0.5))


# ---------------------------------------------------------------------------
# Single-value quantizer (section 3.3 digit maps, section 3.6 plane rule).
# Pinned by the Figure 1 worked example and the closed-form code test.
# ---------------------------------------------------------------------------
def quantize_value(w: float, lo: float, s: float, nbits: int):
    """Quantize one value against a pair (lo, s): returns (q, [b_3..b_N]).

    q is the nearest of the four base levels lo + j*s (ties upward, R1); each
    plane bit is the sign of the residual left by the prefix before it, with
    sign(0) := +1, and moves the reconstruction by +-s/2^(k-1) (Eq. 7).
    """
    w = float(w); lo = float(lo); s = float(s)
    if s == 0.0:
        return 0, [0] * (nbits - 2)
    q = sum(1 for j in range(3) if w - lo >= (j + 0.5) * s)
    rec = lo + s * q
    bits = []
    for k in range(3, nbits + 1):
        b = 1 if w - rec >= 0.0 else 0
        rec += (2 * b - 1) * s / 2.0 ** (k - 1)
        bits.append(b)
    return q, bits


def half_step(s, M: int):
    """t_M = s / 2^(M-1), the half-step of the deepest plane read (Eq. 7)."""
    return s / 2.0 ** (M - 1)


def affine_pair(lo, s, M: int):
    """(lo_M, s_M) of Eq. (10): s_M = s/2^(M-2), lo_M = lo - s(2^(M-2)-1)/2^(M-1)."""
    return lo - s * (2.0 ** (M - 2) - 1.0) / 2.0 ** (M - 1), s / 2.0 ** (M - 2)


# ---------------------------------------------------------------------------
# Encoder (section 3.6 order).  Pinned by hand-worked small matrices in
# tests/golden/encoder_small.json, the Figure 1 example and the invariants.
# ---------------------------------------------------------------------------
# ---------------------------------------------------------------------------
# Codebook metadata (section 3.1, Eq. 5-6, Appendices B and E; readings
# R9-R11).  Pinned by hand-worked tables, the uniform-placement endpoints,
# the symmetric initial pair and an exact-rational brute force of the
# per-group choice.
# ---------------------------------------------------------------------------
def initial_pair(vmin, vmax):
    """The initial pair of Appendix B (never stored): four levels placed
    symmetrically in [min, max], the outer two 6% of the range in from either
    end, so s0 = 0.88 (max - min) / 3 and lo0 = min + 0.06 (max - min)
    (reading R9: the page's "step 0.29 of the range" is this step rounded)."""
    rng = np.asarray(vmax, dtype=np.float64) - np.asarray(vmin, dtype=np.float64)
    return np.asarray(vmin, dtype=np.float64) + 0.06 * rng, 0.88 * rng / 3.0


def uniform_codebooks(lo0, s0):
    """Two 16-entry codebooks placed uniformly over the range of the initial
    pairs (Appendix E's uniform rule): log2 s over [min, max] of log2 s0, and
    lo/s over [min, max] of lo0 / s0, groups with s0 > 0 only; stored as fp16."""
    lo0 = np.asarray(lo0, dtype=np.float64).ravel()
    s0 = np.asarray(s0, dtype=np.float64).ravel()
    pos = s0 > 0.0
    if not pos.any():
        return np.zeros(16, np.float16), np.zeros(16, np.float16)
    L = np.log2(s0[pos])
    P = lo0[pos] / s0[pos]
    t = np.arange(16, dtype=np.float64) / 15.0
    return ((L.min() + t * (L.max() - L.min())).astype(np.float16),
            (P.min() + t * (P.max() - P.min())).astype(np.float16))


def codebook_table(cb_log2s, cb_ratio):
    """The 256 (lo, s) pairs the codebooks span (reading R10): for index
    i * 16 + j, s = fp16(2^cb_log2s[i]) and lo = fp16(cb_ratio[j] * s), each
    computed in float64 from the fp16 inputs and rounded once."""
    L = np.asarray(cb_log2s, dtype=np.float16).astype(np.float64)
    P = np.asarray(cb_ratio, dtype=np.float16).astype(np.float64)
    s = np.exp2(L).astype(np.float16)
    lo = (P[None, :] * s.astype(np.float64)[:, None]).astype(np.float16)
    return lo.reshape(256), np.repeat(s, 16)


def pair_loss(v, lo, s, nbits: int, lam: float = 4.0, E=None):
    """D(lo, s) of Eq. (5) over the last axis of v: the mean over M = 2..N of
    the squared reconstruction errors plus lam times the floor term of Eq. (6),
    rho = s sum_{k=3..N} 2^-(k-1).  E: the calibration mean square E_c of each
    entry's input channel, broadcast against v (None: E_c = 1).  lo, s
    broadcast against v's leading axes."""
    v = np.asarray(v, dtype=np.float64)
    wt = np.ones_like(v) if E is None else np.broadcast_to(np.asarray(E, dtype=np.float64), v.shape)
    lo = np.asarray(lo, dtype=np.float64)[..., None]
    s = np.asarray(s, dtype=np.float64)[..., None]
    d = v - lo
    q = np.zeros(v.shape, dtype=np.float64)
    for j in range(3):
        q += (d >= (j + 0.5) * s)
    q = np.where(s > 0.0, q, 0.0)
    rec = lo + s * q
    rho = s * sum(2.0 ** -(k - 1) for k in range(3, nbits + 1))
    floor = (wt * np.maximum(np.abs(v - rec) - rho, 0.0) ** 2).sum(axis=-1)
    err = (wt * (v - rec) ** 2).sum(axis=-1)
    for k in range(3, nbits + 1):
        b = (v - rec) >= 0.0
        rec = rec + np.where(s > 0.0, (2.0 * b - 1.0) * s / 2.0 ** (k - 1), 0.0)
        err = err + (wt * (v - rec) ** 2).sum(axis=-1)
    return err / (nbits - 1) + lam * floor


def encode(w16: np.ndarray, group: int, nbits: int, frac: float, T: float = 4.0,
           pair_fit: str = "minmax", lam: float = 4.0, post_per_row: int = 0) -> Fields:
    """The reference encoder.  pair_fit "minmax": the pair of R2, stored as two
    fp16 numbers per group.  pair_fit "codebook": the pages' metadata (section
    3.1): codebooks fitted to the initial pairs of Appendix B by uniform
    placement, then per group the index whose (lo, s) minimizes Eq. (5) (E_c = 1,
    lambda = lam) over the group with its pre-grid entry clipped to the next
    value inward (R11); every later step uses the chosen pair.  post_per_row
    = k > 0: the post-grid guard takes the k largest two-bit residuals of every
    row, and the budget caps the pre-grid guard only (R4)."""
    if pair_fit not in ("minmax", "codebook"):
        raise ValueError("pair_fit must be 'minmax' or 'codebook'")
    w16 = np.asarray(w16)
    if w16.ndim != 2 or w16.dtype not in (np.float16, np.float64):
        raise ValueError("encode expects a 2-D float16 (or float64, statistics only) matrix")
    R, C = w16.shape
    if C % group != 0:
        raise ValueError("cols must be a multiple of the group size")
    if nbits < 2:
        raise ValueError("nbits must be >= 2")
    G = C // group
    w = w16.astype(np.float64)                      # exact
    wg = w.reshape(R, G, group)
    flat = np.arange(R * C, dtype=np.int64).reshape(R, G, group)
    K = budget(frac, R, C)
    mask = np.zeros((R, G, group), dtype=bool)

    # 1. Pre-grid guard, ratio criterion (section 3.5, R3).
    mag = np.abs(wg)
    i_max = np.argmax(mag, axis=2)                  # first maximum = lowest column
    a = np.take_along_axis(mag, i_max[..., None], axis=2)[..., 0]
    others = mag.copy()
    np.put_along_axis(others, i_max[..., None], -1.0, axis=2)
    b = others.max(axis=2)
    is_cand = a > T * b
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(b > 0.0, a / np.where(b > 0.0, b, 1.0), np.inf)
    cand_r, cand_g = np.nonzero(is_cand)
    cand_flat = flat[cand_r, cand_g, i_max[cand_r, cand_g]]
    cand_ratio = ratio[cand_r, cand_g]
    order = np.lexsort((cand_flat, -cand_ratio))     # ratio descending, then flat index
    n_pre = min(K, order.shape[0])
    keep = order[:n_pre]
    mask[cand_r[keep], cand_g[keep], i_max[cand_r[keep], cand_g[keep]]] = True

    # 2. Pair fit over the entries that stay in the main stream (R2).
    lo64 = np.where(mask, np.inf, wg).min(axis=2)
    hi64 = np.where(mask, -np.inf, wg).max(axis=2)
    idx = cb_log2s = cb_ratio = None
    if pair_fit == "minmax":
        lo16 = lo64.astype(np.float16)                  # exact for fp16 weights
        s16 = ((hi64 - lo64) / 3.0).astype(np.float16)  # round to nearest even
    else:
        # the group with its pre-grid entry clipped to the next value inward
        # (equal to the min / max of the remaining entries), R11
        v = np.clip(wg, lo64[..., None], hi64[..., None])
        lo0, s0 = initial_pair(lo64, hi64)
        cb_log2s, cb_ratio = uniform_codebooks(lo0, s0)
        tlo, ts = codebook_table(cb_log2s, cb_ratio)
        best = np.full((R, G), np.inf)
        idx = np.zeros((R, G), dtype=np.uint8)
        for c in range(256):                             # lowest index wins ties
            D = pair_loss(v, np.full((R, G), float(tlo[c])), np.full((R, G), float(ts[c])), nbits, lam)
            better = D < best
            best = np.where(better, D, best)
            idx = np.where(better, np.uint8(c), idx)
        lo16, s16 = tlo[idx], ts[idx]
    lo_f = lo16.astype(np.float64)[..., None]
    s_f = s16.astype(np.float64)[..., None]

    # 3. Base code: nearest of lo + j s, ties upward (R1); all entries, including
    #    the pre-grid ones, from their original values (R5); s = 0 -> q = 0 (R7).
    d = wg - lo_f
    q = np.zeros((R, G, group), dtype=np.int64)
    for j in range(3):
        q += (d >= (j + 0.5) * s_f)
    q = np.where(s_f > 0.0, q, 0)

    # 4. Post-grid guard: largest two-bit residuals over the matrix, or the
    #    post_per_row largest of every row (R4).
    r2 = np.abs(wg - (lo_f + s_f * q))
    n_post = 0 if post_per_row else K - n_pre
    if post_per_row > 0:
        m2 = mask.reshape(R, C)                     # a view: writes go to mask
        r2r = r2.reshape(R, C)
        for r in range(R):
            free_cols = np.nonzero(~m2[r])[0]
            order = np.lexsort((free_cols, -r2r[r, free_cols]))[:post_per_row]
            m2[r, free_cols[order]] = True
            n_post += int(order.shape[0])
    if n_post > 0 and not post_per_row:
        free_flat = flat[~mask]                     # ascending flat index
        free_r2 = r2[~mask]
        if n_post >= free_r2.shape[0]:
            pick = free_flat
        else:
            # the n_post-th largest residual; everything above it is taken, and
            # the entries equal to it are taken in flat-index order
            kth = np.partition(free_r2, free_r2.shape[0] - n_post)[free_r2.shape[0] - n_post]
            above = free_r2 > kth
            ties = np.nonzero(free_r2 == kth)[0][: n_post - int(above.sum())]
            pick = np.concatenate([free_flat[above], free_flat[ties]])
        mask.reshape(-1)[pick] = True

    # 5. Planes: sign of the residual of the preceding prefix (sections 3.3, 3.6);
    #    skipped (0) at held-out positions and in zero-step groups (R5, R7).
    planes = np.zeros((nbits - 2, R, G, group), dtype=np.uint8)
    rec = lo_f + s_f * q
    active = (~mask) & (s_f > 0.0)
    for k in range(3, nbits + 1):
        bk = ((wg - rec) >= 0.0) & active
        planes[k - 3] = bk
        rec = rec + np.where(active, (2.0 * bk - 1.0) * s_f / 2.0 ** (k - 1), 0.0)

    # 6. Side record as CSR sorted by (row, col), the recorded value = w (R6).
    mask2 = mask.reshape(R, C)
    rr, cc = np.nonzero(mask2)                      # row-major order = (row, col) sorted
    row_ptr = np.zeros(R + 1, dtype=np.int64)
    np.add.at(row_ptr, rr + 1, 1)
    row_ptr = np.cumsum(row_ptr).astype(np.int32)
    return Fields(
        rows=R, cols=C, group=group, nbits=nbits,
        q=q.reshape(R, C).astype(np.uint8),
        planes=planes.reshape(nbits - 2, R, C),
        lo=lo16, s=s16, mask=mask2,
        row_ptr=row_ptr, col=cc.astype(np.int32), val=w16[rr, cc].astype(np.float16),
        n_pre=int(n_pre), n_post=int(max(n_post, 0)),
        idx=idx, cb_log2s=cb_log2s, cb_ratio=cb_ratio,
    )


# ---------------------------------------------------------------------------
# Decode.  codes(): Eq. (8), pinned by Figure 1, the prefix property and the
# closed-form code.  w_main(): Eq. (9), pinned by Eq. (10) (exhaustive, exact
# rationals), the midpoint property (Appendix C, Eq. 12), the error bound t_M,
# the reach rho (Eq. 6) and the textbook INT2 special case.
# ---------------------------------------------------------------------------
def _check_bits(F: Fields, M: int):
    if not (2 <= M <= F.nbits):
        raise ValueError(f"bits must be in [2, {F.nbits}]")


def codes(F: Fields, M: int) -> np.ndarray:
    """Composite integer u_M = q 2^(M-2) + sum_{k=3..M} b_k 2^(M-k) (Eq. 8), uint8 [R, C]."""
    _check_bits(F, M)
    u = F.q.astype(np.int64) << (M - 2)
    for k in range(3, M + 1):
        u += F.planes[k - 3].astype(np.int64) << (M - k)
    return u.astype(np.uint8)


def _expand(F: Fields, a: np.ndarray) -> np.ndarray:
    return np.repeat(a.astype(np.float64), F.group, axis=1)


def w_main(F: Fields, M: int, rows: Optional[slice] = None) -> np.ndarray:
    """Main-stream reconstruction lo + s q + sum (2 b_k - 1) s/2^(k-1) (Eq. 9), float64."""
    _check_bits(F, M)
    sl = rows if rows is not None else slice(None)
    lo = _expand(F, F.lo[sl])
    s = _expand(F, F.s[sl])
    w = lo + s * F.q[sl].astype(np.float64)
    for k in range(3, M + 1):
        w += (2.0 * F.planes[k - 3][sl].astype(np.float64) - 1.0) * s / 2.0 ** (k - 1)
    return w


def w_hat(F: Fields, M: int, rows: Optional[slice] = None) -> np.ndarray:
    """Complete reconstruction (1 - m) W_main + P (Eq. 4), float64."""
    sl = rows if rows is not None else slice(None)
    wm = w_main(F, M, sl)
    m = F.mask[sl]
    start = 0 if sl.start is None else sl.start
    stop = F.rows if sl.stop is None else sl.stop
    P = np.zeros_like(wm)
    lo_e, hi_e = int(F.row_ptr[start]), int(F.row_ptr[stop])
    rr = np.repeat(np.arange(start, stop), np.diff(F.row_ptr[start:stop + 1]))
    P[rr - start, F.col[lo_e:hi_e]] = F.val[lo_e:hi_e].astype(np.float64)
    return np.where(m, P, wm)


def gemv(F: Fields, x16: np.ndarray, M: int, block_rows: int = 8192) -> np.ndarray:
    """y = W_hat^(M) x in float64 (streams row blocks to bound memory)."""
    x = np.asarray(x16).astype(np.float64)
    if x.shape != (F.cols,):
        raise ValueError("x must have shape [cols]")
    y = np.empty(F.rows, dtype=np.float64)
    for r0 in range(0, F.rows, block_rows):
        r1 = min(F.rows, r0 + block_rows)
        y[r0:r1] = w_hat(F, M, slice(r0, r1)) @ x
    return y


# ---------------------------------------------------------------------------
# Run-time inverse AWQ scale (section 3.6 and Appendix E; reading R8).
# Pinned by: unit scale gives x back, power-of-two scales scale y exactly, a
# single scaled channel changes y by that column alone, and round-to-nearest
# on hand-picked fp16 products.
# ---------------------------------------------------------------------------
def scale_x(x16: np.ndarray, inv_scale16: np.ndarray) -> np.ndarray:
    """x'_c = fp16(x_c * inv_scale_c): the float64 product of two fp16 numbers
    is exact, so casting it to fp16 rounds once, to nearest even."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    a = np.asarray(inv_scale16, dtype=np.float16).astype(np.float64)
    if x.shape != a.shape:
        raise ValueError("x and the scale must have the same shape")
    return (x * a).astype(np.float16)


def gemv_scaled(F: Fields, x16: np.ndarray, inv_scale16: np.ndarray, M: int) -> np.ndarray:
    """y = W_hat^(M) fp16(x * inv_scale) in float64."""
    return gemv(F, scale_x(x16, inv_scale16), M)
