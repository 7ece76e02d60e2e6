"""Pins of the oracle's inference from packed factors, y = B diag(D) C x (ExTernD review,
Significance: ternary additions and subtractions plus one scale per component).

The oracle is checked against (1) the dense product of the unpacked factors in fp64 (numpy
matmuls, an independent route through the packing), (2) an exact special case, and (3) the
decomposition's own energy bound |A x - y| <= |R|_F |x|, |R|_F^2 = (1 - energy) |A|_F^2."""

import numpy as np
import pytest

import oracle
from expanded_rank_matrix_amd import inputs



def pack(T):
    """int8 {-1, 0, 1} rows -> packed 2-bit words (00 = 0, 01 = +1, 11 = -1)."""
    T = np.asarray(T)
    L = T.shape[1]
    w = (L + 15) // 16
    codes = np.where(T == 0, 0, np.where(T > 0, 1, 3)).astype(np.uint32)
    codes = np.pad(codes, ((0, 0), (0, w * 16 - L)))
    shifts = (2 * np.arange(16, dtype=np.uint32))[None, None, :]
    return (codes.reshape(T.shape[0], w, 16) << shifts).sum(axis=2, dtype=np.uint64).astype(np.uint32)


def random_factors(rng, k, m, n, density=0.55):
    Bt = rng.choice([-1, 0, 1], size=(k, m), p=[density / 2, 1 - density, density / 2]).astype(np.int8)
    Ct = rng.choice([-1, 0, 1], size=(k, n), p=[density / 2, 1 - density, density / 2]).astype(np.int8)
    D = rng.standard_normal(k).astype(np.float32)
    return Bt, Ct, D


@pytest.mark.parametrize("k,m,n,batch", [(1, 1, 1, 1), (5, 7, 9, 2), (64, 17, 33, 3), (300, 389, 103, 2)])
def test_apply_matches_dense_product(k, m, n, batch):
    rng = np.random.default_rng(k + m + n)
    Bt, Ct, D = random_factors(rng, k, m, n)
    X = rng.standard_normal((batch, n)).astype(np.float32)
    Y = oracle.apply(pack(Bt), pack(Ct), D, m, n, X)
    S = (Ct.astype(np.float64) @ X.T.astype(np.float64)) * D.astype(np.float64)[:, None]  # k x batch
    ref = (Bt.T.astype(np.float64) @ S).T                                                 # batch x m
    # one fp32 rounding of an fp64 sum: within an fp32 ulp of the exact value (plus fp64 noise)
    bound = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) + 1e-12 * np.abs(Bt.T.astype(np.float64) @ np.abs(S)).T
    assert np.all(np.abs(Y.astype(np.float64) - ref) <= bound)


def test_apply_identity_factors_scale_exactly():
    n = 37
    eye = np.eye(n, dtype=np.int8)
    D = np.linspace(-2, 2, n).astype(np.float32)
    x = np.random.default_rng(1).standard_normal(n).astype(np.float32)
    y = oracle.apply(pack(eye), pack(eye), D, n, n, x)
    np.testing.assert_array_equal(y, (D.astype(np.float64) * x.astype(np.float64)).astype(np.float32))
    # sign flips in B only negate
    y2 = oracle.apply(pack(-eye), pack(eye), D, n, n, x)
    np.testing.assert_array_equal(y2, -y)


def test_apply_of_a_decomposition_within_its_energy_bound():
    A, h = inputs.make_input("tiny64x48")
    m, n = A.shape
    r = oracle.decompose(A, 3.0, 0.0, None, 4, 1)
    k = len(r["D"])
    X = np.random.default_rng(5).standard_normal((4, n)).astype(np.float32)
    Y = oracle.apply(r["B"].reshape(k, -1), r["C"].reshape(k, -1), r["D"], m, n, X)
    AX = X.astype(np.float64) @ A.T.astype(np.float64)
    resid_fro = np.sqrt(max(0.0, 1.0 - r["energy"][-1])) * np.linalg.norm(A.astype(np.float64))
    err = np.linalg.norm(AX - Y, axis=1)
    assert np.all(err <= resid_fro * np.linalg.norm(X, axis=1) * (1 + 1e-6) + 1e-5)
    assert r["energy"][-1] > 0.9
