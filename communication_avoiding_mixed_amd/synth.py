"""Seeded synthetic workloads for CA-SGD on generalized linear models.

This module only draws data: it holds none of the method's arithmetic (no
rounding to low precision, no sampling of minibatches, no losses).  Both the
HIP path and the CPU oracle take its float32 arrays as their common input.

The workloads follow the shapes of the data sets named in the Abstract of
"Mixed-Precision Communication-Avoiding SGD for Generalized Linear Models on
GPUs" (epsilon, SUSY, HIGGS, synth, Poisson-synth) plus one small logistic
case.  The real data sets are not available here; these stand in for them with
the same row and column counts and a comparable value structure.  The page
gives no shape for SUSY: it is taken as the public data set's 5,000,000 rows of
18 features, run with the HIGGS-shaped case's s, b and eta (both are tall,
narrow logistic problems).

Recipe (all draws from numpy's PCG64 generator seeded with `seed`, in this
order: X as float32, then w* as float64, then noise / label flips / counts):

  logistic-4096x64  X ~ N(0, 1/64); y = sign(X w*) with 5% of labels flipped
  epsilon           X ~ N(0, 1), each row scaled to unit L2 norm (norm taken in
                    float64); y = sign(X w*) with 10% flipped
  higgs             even columns N(0, 1), odd columns lognormal(0, 0.5), each
                    column standardised (float64 mean, population std);
                    y = sign(X w*) with 25% flipped
  susy              columns 0-7 N(0, 1), columns 8-17 lognormal(0, 0.5), each
                    column standardised as for higgs; y = sign(X w*) with 20%
                    flipped
  synth-lsq         X ~ N(0, 1/512); y = X w* + N(0, 0.01^2)
  poisson-synth     X ~ 0.5 * N(0, 1/256); y ~ Poisson(exp(X w*))

w* ~ N(0, I) in every case, labels are computed in float64 from the float32 X,
and sign(0) = +1.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    m: int
    n: int
    s: int
    b: int
    eta: float
    loss: str
    outer: int
    storage: str = "bf16"
    # scale of the seeded starting weights used by single-step parity tests,
    # chosen so that margins x . w0 are about N(0, 1)
    w0_scale: float = 1.0


WORKLOADS = {
    "logistic-4096x64": Workload("logistic-4096x64", 4096, 64, 4, 16, 0.5, "logistic", 20),
    "epsilon": Workload("epsilon", 400_000, 2000, 16, 64, 1.0, "logistic", 200),
    "higgs": Workload("higgs", 11_000_000, 28, 32, 128, 0.1, "logistic", 200,
                      w0_scale=float(1.0 / np.sqrt(28.0))),
    "susy": Workload("susy", 5_000_000, 18, 32, 128, 0.1, "logistic", 200,
                     w0_scale=float(1.0 / np.sqrt(18.0))),
    "synth-lsq": Workload("synth-lsq", 1_000_000, 512, 8, 256, 0.05, "squared", 200),
    "poisson-synth": Workload("poisson-synth", 2_000_000, 256, 16, 128, 0.01, "poisson", 200),
}

_CHUNK = 1 << 13


def _matvec64(X, w):
    """X (float32) @ w (float64) in float64, a chunk of rows at a time."""
    out = np.empty(X.shape[0], dtype=np.float64)
    for a in range(0, X.shape[0], _CHUNK):
        out[a:a + _CHUNK] = X[a:a + _CHUNK].astype(np.float64) @ w
    return out


def _signs_with_flips(rng, margins, flip_rate):
    y = np.where(margins >= 0.0, 1.0, -1.0)
    flip = rng.random(margins.shape[0]) < flip_rate
    return np.where(flip, -y, y).astype(np.float32)


def make_data(name: str, seed: int = 0, m: int | None = None):
    """Return (X float32 [m, n] C-contiguous, y float32 [m]) for a workload.

    `m` overrides the row count (same recipe, fewer rows) for small tests.
    """
    wl = WORKLOADS[name]
    m = wl.m if m is None else int(m)
    n = wl.n
    rng = np.random.Generator(np.random.PCG64(seed))

    if name == "logistic-4096x64":
        X = rng.standard_normal((m, n), dtype=np.float32) * np.float32(1.0 / 8.0)
    elif name == "epsilon":
        X = rng.standard_normal((m, n), dtype=np.float32)
        for a in range(0, m, _CHUNK):
            Xc = X[a:a + _CHUNK].astype(np.float64)
            Xc /= np.sqrt(np.sum(Xc * Xc, axis=1))[:, None]
            X[a:a + _CHUNK] = Xc.astype(np.float32)
    elif name in ("higgs", "susy"):
        X = np.empty((m, n), dtype=np.float32)
        if name == "higgs":
            normal, skewed = np.arange(0, n, 2), np.arange(1, n, 2)
        else:
            normal, skewed = np.arange(0, 8), np.arange(8, n)
        X[:, normal] = rng.standard_normal((m, normal.size), dtype=np.float32)
        X[:, skewed] = rng.lognormal(0.0, 0.5, (m, skewed.size)).astype(np.float32)
        for c in range(n):
            col = X[:, c].astype(np.float64)
            mu = col.mean()
            sd = np.sqrt(np.mean((col - mu) ** 2))
            X[:, c] = ((col - mu) / sd).astype(np.float32)
    elif name == "synth-lsq":
        X = rng.standard_normal((m, n), dtype=np.float32) * np.float32(1.0 / np.sqrt(512.0))
    elif name == "poisson-synth":
        X = rng.standard_normal((m, n), dtype=np.float32) * np.float32(0.5 / 16.0)
    else:
        raise KeyError(name)
    X = np.ascontiguousarray(X, dtype=np.float32)

    w_star = rng.standard_normal(n)
    margins = _matvec64(X, w_star)
    if name == "logistic-4096x64":
        y = _signs_with_flips(rng, margins, 0.05)
    elif name == "epsilon":
        y = _signs_with_flips(rng, margins, 0.10)
    elif name == "higgs":
        y = _signs_with_flips(rng, margins, 0.25)
    elif name == "susy":
        y = _signs_with_flips(rng, margins, 0.20)
    elif name == "synth-lsq":
        y = (margins + 0.01 * rng.standard_normal(m)).astype(np.float32)
    else:
        y = rng.poisson(np.exp(margins)).astype(np.float32)
    return X, y


def make_w0(name: str, seed: int, n: int | None = None) -> np.ndarray:
    """Seeded float32 starting weights with margins of order one."""
    wl = WORKLOADS[name]
    n = wl.n if n is None else n
    rng = np.random.Generator(np.random.PCG64(0x5EED0000 + seed))
    return (rng.standard_normal(n) * wl.w0_scale).astype(np.float32)


def make_uniform(shape, seed: int, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    """Seeded float32 values uniform in [lo, hi) for edge-case tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def make_grid(shape, seed: int, kmax: int, scale_log2: int) -> np.ndarray:
    """Seeded float32 values k * 2^-scale_log2, k uniform in [-kmax, kmax].

    Values with few significant bits: products and sums of them stay exact
    in float32 as long as the sums stay below 2^24 grid units, so a dot
    product comes out the same in any summation order.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    k = rng.integers(-kmax, kmax + 1, size=shape)
    return (k.astype(np.float64) * 2.0 ** -scale_log2).astype(np.float32)
