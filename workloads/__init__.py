"""Seeded synthetic inputs for the StagQ batch-one GEMV workloads.

This module only draws random numbers: it holds none of the quantization
method's arithmetic.  The oracle (test infrastructure) and the product path
(the HIP library, the benchmark) both take their weights and activations from
here, so the two sides see identical inputs.

Workloads follow the matrix shapes of the StagQ paper's kernel evaluation
(Appendix F, Table 8: Llama-3-8B and Phi-4 projections, written there as
input x output; here every shape is rows(out) x cols(in)).  The paper times
its kernel on synthetic weights without giving their distribution, so the
value distributions below are this project's choice:

* "normal_outliers": N(0, 0.02^2), then round(0.005*R*C) positions drawn
  uniformly without replacement are scaled by 10 before the fp16 cast.
* "student_t": Student-t with nu = 4 scaled to standard deviation 0.02,
  i.e. 0.02 * t / sqrt(2) (the variance of t_4 is 2).

Within one matrix the draw order is fixed: W, then the outlier positions (if
any), then x ~ N(0, 1); everything is drawn in float64 and rounded to fp16.

synth_channel_energy() stands in for the calibration mean square E_c of each
input channel, which the paper measures on C4 text (not available here): a
log-normal spread, E_c = exp(z), z ~ N(0, 1), with round(0.005 * C) channels
(at least one) drawn without replacement and scaled by 100, the few
large-activation channels such models show.  It has its own generator, so it
leaves the W and x draws unchanged.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Tuple

import numpy as np

__all__ = ["Matrix", "Workload", "WORKLOADS", "synth_matrix", "synth_channel_energy", "array_digest"]


@dataclass(frozen=True)
class Matrix:
    name: str
    rows: int
    cols: int
    seed: int


@dataclass(frozen=True)
class Workload:
    name: str
    matrices: Tuple[Matrix, ...]
    dist: str
    group: int
    nbits: int          # N: base + (N - 2) refinement planes
    frac: float         # side-record budget as a fraction of R*C
    bits: Tuple[int, ...]
    ratio_T: float = 4.0
    note: str = field(default="")
    post_per_row: int = 0   # k > 0: k post-grid entries per row (frac caps the pre-grid guard)


WORKLOADS = {
    "tiny": Workload(
        "tiny", (Matrix("W", 256, 512, 0),), "normal_outliers", 64, 4, 0.005, (2, 3, 4),
        note="256x512, N(0,0.02) with 0.5% outliers at 10x, g=64"),
    "attn": Workload(
        "attn", (Matrix("qkvo", 4096, 4096, 0),), "student_t", 128, 4, 0.001, (2, 3, 4),
        note="Llama-3.1-8B attention projection 4096x4096"),
    "mlp": Workload(
        "mlp", (Matrix("gate_up", 14336, 4096, 0), Matrix("down", 4096, 14336, 1)),
        "student_t", 128, 4, 0.001, (2, 3, 4),
        note="Llama-3.1-8B MLP: gate/up 14336x4096, down 4096x14336"),
    "mlp_rows": Workload(
        "mlp_rows", (Matrix("gate_up", 14336, 4096, 0), Matrix("down", 4096, 14336, 1)),
        "student_t", 128, 4, 0.001, (2, 3, 4),
        note="the MLP shapes with 4 post-grid entries per row (about the same side-record size "
             "as 0.1% of the weights), the record in fixed per-row slots or CSR",
        post_per_row=4),
    "phi4_mlp": Workload(
        "phi4_mlp", (Matrix("gate_up", 17920, 5120, 0), Matrix("down", 5120, 17920, 1)),
        "student_t", 128, 6, 0.002, (2, 3, 4, 5, 6),
        note="Phi-4 MLP: 17920x5120 and 5120x17920, base + 4 planes"),
    "layer_sweep": Workload(
        "layer_sweep",
        (Matrix("q", 4096, 4096, 0), Matrix("k", 1024, 4096, 1), Matrix("v", 1024, 4096, 2),
         Matrix("o", 4096, 4096, 3), Matrix("gate", 14336, 4096, 4), Matrix("up", 14336, 4096, 5),
         Matrix("down", 4096, 14336, 6), Matrix("lm_head", 128256, 4096, 7)),
        "student_t", 128, 4, 0.001, (2, 3, 4),
        note="8B-style decoder layer + LM head, bits switched per call"),
}


def _draw_w(rng: np.random.Generator, rows: int, cols: int, dist: str) -> np.ndarray:
    if dist == "normal_outliers":
        w = rng.normal(0.0, 0.02, size=(rows, cols))
        n_out = int(np.floor(0.005 * rows * cols + 0.5))
        pos = rng.choice(rows * cols, size=n_out, replace=False)
        w.reshape(-1)[pos] *= 10.0
        return w
    if dist == "student_t":
        return 0.02 * rng.standard_t(4.0, size=(rows, cols)) / np.sqrt(2.0)
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=(rows, cols))
    raise ValueError(f"unknown distribution {dist!r}")


def synth_matrix(rows: int, cols: int, dist: str, seed: int):
    """Return (W fp16 [rows, cols], x fp16 [cols]) for one matrix of a workload."""
    rng = np.random.default_rng(seed)
    w = _draw_w(rng, rows, cols, dist).astype(np.float16)
    x = rng.standard_normal(cols).astype(np.float16)
    return w, x


def synth_channel_energy(cols: int, seed: int) -> np.ndarray:
    """E_c > 0 for every input channel (float64 [cols]), drawn as described above."""
    rng = np.random.default_rng([seed, 7])
    e = np.exp(rng.standard_normal(cols))
    n_big = max(1, int(np.floor(0.005 * cols + 0.5)))
    e[rng.choice(cols, size=n_big, replace=False)] *= 100.0
    return e


def array_digest(a: np.ndarray) -> str:
    """Short content hash of an array (dtype, shape and bytes)."""
    h = hashlib.sha256()
    h.update(str(a.dtype).encode())
    h.update(str(a.shape).encode())
    h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:16]
