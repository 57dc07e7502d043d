"""Seeded synthetic workloads for the blocked vocabulary-projection cross-entropy.

This module is shared by the tests, the benchmark and the smoke check. It draws
inputs only: it contains none of the method's arithmetic (no logits, no
log-sum-exp, no gradients), so the CPU oracle and the HIP path stay independent
of each other and meet only through the arrays produced here.

Shapes follow the five workloads the operator is measured on (the output head
of the MoE models in "Flattening Every Memory Peak in Long-Context
Mixture-of-Experts Training", section 3.2 "Ring-DTP"): H holds the final hidden
states of the tokens resident on one rank, W the vocabulary projection, and the
labels the next-token targets.

Recipe (every stream is independent, derived from one seed):
  SeedSequence(seed).spawn(6) -> streams for H, W, labels, vocab permutation,
  ignored positions, outlier rows; each stream is a numpy ``default_rng``.
  * H ~ N(0, 1) drawn as float32; rows chosen as outliers are multiplied by the
    outlier scale in float32; then H is rounded once to bfloat16
    (round-to-nearest-even) unless the workload is float32.
  * W ~ N(0, sigma^2) drawn as float32 standard normals times sigma, then
    rounded once to bfloat16 (same rule).
  * labels: uniform integers in [0, V), or a finite Zipf law p_k ~ k^-s over
    ranks k = 1..V sampled by inverse CDF, mapped through a random permutation
    of the vocabulary.
  * an exact count round(p * N) of positions, drawn without replacement, is set
    to the ignore index.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

IGNORE_INDEX = -100


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    N: int            # tokens resident on the rank
    d: int            # hidden width
    V: int            # vocabulary size
    R: int            # number of vocabulary shards (ring degree)
    dtype: str        # "bf16" or "f32": storage type of H and W
    w_std: float      # standard deviation of W's entries
    labels: str       # "uniform" or "zipf"
    zipf_s: float = 0.0
    ignore_frac: float = 0.0
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0

    @property
    def n_ignored(self) -> int:
        return int(round(self.ignore_frac * self.N))

    @property
    def n_outliers(self) -> int:
        return int(round(self.outlier_frac * self.N))

    def flops(self) -> float:
        """Forward + backward-with-recompute multiply-add work: 8*N*d*V."""
        return 8.0 * self.N * self.d * self.V


# The five workloads. The logit standard deviation of the 1M-context slice is 3,
# obtained with H ~ N(0,1) and W's std = 3 / sqrt(d).
WORKLOADS = [
    Workload("tiny_f32", N=128, d=64, V=1024, R=1, dtype="f32", w_std=0.02,
             labels="uniform"),
    Workload("n4k_d2k_v32k_r4", N=4096, d=2048, V=32000, R=4, dtype="bf16",
             w_std=0.02, labels="uniform", ignore_frac=0.05),
    Workload("n16k_d4k_v128k_r8", N=16384, d=4096, V=128256, R=8,
             dtype="bf16", w_std=0.02, labels="zipf", zipf_s=1.1,
             ignore_frac=0.02),
    Workload("ctx1m_slice_n64k_d7168_v129k_r8", N=65536, d=7168, V=129280,
             R=8, dtype="bf16", w_std=3.0 / math.sqrt(7168), labels="zipf",
             zipf_s=1.1, ignore_frac=0.02),
    Workload("stress_n128k_d5120_v152k_r7", N=131072, d=5120, V=151936, R=7,
             dtype="bf16", w_std=0.02, labels="zipf", zipf_s=1.2,
             ignore_frac=0.10, outlier_frac=0.01, outlier_scale=20.0),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def custom(N, d, V, R, dtype="bf16", w_std=0.02, labels="uniform", zipf_s=1.1,
           ignore_frac=0.0, outlier_frac=0.0, outlier_scale=1.0,
           name="custom") -> Workload:
    return Workload(name, N, d, V, R, dtype, w_std, labels, zipf_s,
                    ignore_frac, outlier_frac, outlier_scale)


# ----------------------------------------------------------------------------
# bfloat16 storage helpers (bit manipulation only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 with round-to-nearest-even; returns uint16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# generation
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Inputs:
    """Host arrays. For bf16 workloads H and W are uint16 bit patterns."""
    workload: Workload
    H: np.ndarray
    W: np.ndarray
    labels: np.ndarray   # int64 [N]
    outlier_rows: np.ndarray

    def H_f64(self, rows=None) -> np.ndarray:
        h = self.H if rows is None else self.H[rows]
        if self.workload.dtype == "bf16":
            return bf16_bits_to_f32(h).astype(np.float64)
        return h.astype(np.float64)

    def W_f64(self, rows=None) -> np.ndarray:
        w = self.W if rows is None else self.W[rows]
        if self.workload.dtype == "bf16":
            return bf16_bits_to_f32(w).astype(np.float64)
        return w.astype(np.float64)


def _streams(seed: int):
    ss = np.random.SeedSequence(seed).spawn(6)
    return [np.random.default_rng(s) for s in ss]


def _normal_matrix(rng, rows, cols, scale, bf16, row_scale=None,
                   chunk_rows=4096):
    """rows x cols standard normals * scale, drawn in row chunks from one
    stream (the stream's output does not depend on the chunking)."""
    out = np.empty((rows, cols), dtype=np.uint16 if bf16 else np.float32)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = rng.standard_normal((r1 - r0) * cols, dtype=np.float32)
        x = x.reshape(r1 - r0, cols)
        if scale != 1.0:
            x *= np.float32(scale)
        if row_scale is not None:
            x *= row_scale[r0:r1, None]
        out[r0:r1] = f32_to_bf16_bits(x) if bf16 else x
    return out


def zipf_cdf(V: int, s: float) -> np.ndarray:
    k = np.arange(1, V + 1, dtype=np.float64)
    p = k ** (-s)
    c = np.cumsum(p)
    return c / c[-1]


def make_labels(w: Workload, rng_lab, rng_perm, rng_ign) -> np.ndarray:
    N, V = w.N, w.V
    if w.labels == "uniform":
        lab = rng_lab.integers(0, V, size=N, dtype=np.int64)
    elif w.labels == "zipf":
        cdf = zipf_cdf(V, w.zipf_s)
        u = rng_lab.random(N)
        rank = np.searchsorted(cdf, u, side="right")
        rank = np.minimum(rank, V - 1)
        perm = rng_perm.permutation(V).astype(np.int64)
        lab = perm[rank]
    else:
        raise ValueError(w.labels)
    n_ign = w.n_ignored
    if n_ign:
        pos = rng_ign.choice(N, size=n_ign, replace=False)
        lab[pos] = IGNORE_INDEX
    return lab


def make_inputs(w: Workload, seed: int = 0) -> Inputs:
    rH, rW, rLab, rPerm, rIgn, rOut = _streams(seed)
    bf16 = w.dtype == "bf16"
    outl = np.zeros(0, dtype=np.int64)
    row_scale = None
    if w.n_outliers:
        outl = np.sort(rOut.choice(w.N, size=w.n_outliers, replace=False))
        row_scale = np.ones(w.N, dtype=np.float32)
        row_scale[outl] = np.float32(w.outlier_scale)
    H = _normal_matrix(rH, w.N, w.d, 1.0, bf16, row_scale)
    W = _normal_matrix(rW, w.V, w.d, w.w_std, bf16)
    lab = make_labels(w, rLab, rPerm, rIgn)
    return Inputs(w, H, W, lab, outl)


def fingerprint(inp: Inputs, stride: int = 997) -> str:
    """sha256 over the shapes, every ``stride``-th row of H and W (from row
    0), the labels and the outlier rows: identifies a seeded input set, so
    that values stored from one generation are used only with the same
    inputs."""
    import hashlib
    w = inp.workload
    h = hashlib.sha256()
    h.update(repr((w.N, w.d, w.V, w.dtype)).encode())
    for a in (inp.H[::stride], inp.W[::stride], inp.labels,
              inp.outlier_rows):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()
