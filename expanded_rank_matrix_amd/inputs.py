"""Seeded synthetic inputs for the decomposition engine.

This module only draws random matrices and weights; it holds none of the method's arithmetic.
Both the GPU path and the CPU oracle are fed from it.

The pages measure real weight matrices of small open models (shapes up to about 9216 x 2560,
hidden size 2560, MLP width 9728) with llama.cpp imatrix statistics as importance weights
(ExTernD review, Validation and Limitations; pith.science, assumptions).  Neither the weights
nor the statistics are available, so heavy-tailed Student-t matrices of those shapes, with
outlier columns, and log-normal column weights stand in for them.

All draws use numpy's PCG64 (``default_rng(seed)``) in fp64, row-major, then cast to fp32.
A Student-t matrix "at std s" is ``s / sqrt(nu / (nu - 2)) * standard_t(nu)``.
"""

from __future__ import annotations

import numpy as np

# name -> workload.  m, n, mu, tau, als_iters, block as passed to externd_decompose.
CONFIGS = {
    # Tiny oracle case: iid N(0,1), sequential, 4 ALS iterations.
    "tiny64x48": dict(m=64, n=48, mu=2.0, tau=0.0, als_iters=4, block=1, seed=0,
                      kind="normal"),
    # 1024 x 1024 Student-t plus a rank-16 Gaussian term holding 30% of the energy.
    "lowrank1024": dict(m=1024, n=1024, mu=1.5, tau=0.1, als_iters=4, block=1, seed=1,
                        kind="t_lowrank", nu=4.0, std=0.02, rank=16, share=0.3),
    # Attention-projection shape: 2560 x 2560, 8 outlier columns x20, mu = 3.
    "attn2560": dict(m=2560, n=2560, mu=3.0, tau=0.0, als_iters=4, block=1, seed=2,
                     kind="t_outliers", nu=4.0, std=0.02, outliers=8, scale=20.0),
    # MLP up/gate shape: 9728 x 2560, block-ALS b = 64.
    "mlp9728x2560": dict(m=9728, n=2560, mu=2.0, tau=0.3, als_iters=3, block=64, seed=3,
                         kind="t", nu=5.0, std=0.015),
    # Importance-weighted down projection: 2560 x 9728, block-ALS b = 128, log-normal weights.
    "down2560x9728": dict(m=2560, n=9728, mu=3.0, tau=0.2, als_iters=3, block=128, seed=4,
                          kind="t", nu=4.0, std=0.015, weights="lognormal"),
}


def student_t(rng: np.random.Generator, shape, nu: float, std: float) -> np.ndarray:
    return (std / np.sqrt(nu / (nu - 2.0))) * rng.standard_t(nu, size=shape)


def make_matrix(m: int, n: int, seed: int, kind: str = "normal", nu: float = 4.0,
                std: float = 0.02, rank: int = 16, share: float = 0.3, outliers: int = 8,
                scale: float = 20.0, weights: str | None = None):
    """Draw A (m x n, fp32) and optional column weights h (n, fp32).  A is drawn first."""
    rng = np.random.default_rng(seed)
    if kind == "normal":
        A = rng.standard_normal((m, n))
    elif kind == "t":
        A = student_t(rng, (m, n), nu, std)
    elif kind == "t_lowrank":
        N = student_t(rng, (m, n), nu, std)
        G1 = rng.standard_normal((m, rank))
        G2 = rng.standard_normal((n, rank))
        L = G1 @ G2.T
        alpha = np.sqrt((share / (1.0 - share)) * np.sum(N * N) / np.sum(L * L))
        A = N + alpha * L
    elif kind == "t_outliers":
        A = student_t(rng, (m, n), nu, std)
        cols = np.sort(rng.choice(n, size=min(outliers, n), replace=False))
        A[:, cols] *= scale
    else:
        raise ValueError(kind)
    h = None
    if weights == "lognormal":
        h = np.exp(rng.standard_normal(n))
        h = h / np.mean(h)
        h = h.astype(np.float32)
    return np.ascontiguousarray(A.astype(np.float32)), h


def make_input(name: str, m: int | None = None, n: int | None = None, seed: int | None = None):
    """The named workload's (A, h); m, n or seed may be overridden for scaled-down cases that
    keep the workload's value distribution."""
    c = dict(CONFIGS[name])
    mm = c["m"] if m is None else m
    nn = c["n"] if n is None else n
    sd = c["seed"] if seed is None else seed
    kw = {k: c[k] for k in ("nu", "std", "rank", "share", "outliers", "scale", "weights") if k in c}
    return make_matrix(mm, nn, sd, c["kind"], **kw)


def random_vectors(seed: int, count: int, length: int) -> np.ndarray:
    """count x length iid N(0,1) vectors, fp32."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((count, length)).astype(np.float32)


def lognormal_weights(seed: int, length: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    h = np.exp(rng.standard_normal(length))
    return (h / np.mean(h)).astype(np.float32)
