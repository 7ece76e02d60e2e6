"""GPU parity of inference from the packed factors (externd_apply_factors, through the C ABI)
against the oracle: y = B diag(D) C x, one fp32 rounding of each output.  The oracle sums in fp64
in index order; the GPU forms both sums exactly over fixed-point images of x (per vector, at most
50 bits and n |image| <= 2^62) and of s = D (C x) (at most 50 bits and k |image| <= 2^62).  The
bar, derived from that arithmetic: the two may differ by the images' rounding,
  sum_i |B_ri D_i| nnz(C_i) 2^(E_x - P_x - 1) + nnz(B_r) 2^(E_s - P_s - 1)
(2^E bounds the vector's max |x| or |s|, P is the image's bit count), plus two fp32 ulps of the
output and 1e-12 of the sum of the magnitudes of the terms (the fp64 roundings on both sides)."""

import numpy as np
import pytest
import torch

import expanded_rank_matrix_amd as erm
import oracle
from expanded_rank_matrix_amd import inputs
from tests.test_oracle_apply import pack, random_factors

pytestmark = pytest.mark.gpu


def gpu_apply(Bp, Cp, D, m, n, X):
    dev = torch.device("cuda:0")
    B = torch.from_numpy(np.ascontiguousarray(Bp).view(np.int32)).to(dev)
    C = torch.from_numpy(np.ascontiguousarray(Cp).view(np.int32)).to(dev)
    Dt = torch.from_numpy(np.ascontiguousarray(D, dtype=np.float32)).to(dev)
    Xt = torch.from_numpy(np.ascontiguousarray(X, dtype=np.float32)).to(dev)
    Y = erm.apply_factors(B, C, Dt, m, n, Xt)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def check(Bt, Ct, D, X, label):
    m, n = Bt.shape[1], Ct.shape[1]
    Bp, Cp = pack(Bt), pack(Ct)
    Yg = gpu_apply(Bp, Cp, D, m, n, X)
    Yo = oracle.apply(Bp, Cp, D, m, n, X)
    k = Bt.shape[0]
    Bd, Cd, Dd = Bt.astype(np.float64), Ct.astype(np.float64), D.astype(np.float64)
    Sv = (Cd @ X.T.astype(np.float64)) * Dd[:, None]  # k x batch
    mag = (np.abs(Bd.T) @ np.abs(Sv)).T
    bits = lambda length: min(50, 62 - int(length).bit_length())
    ex = np.array([np.frexp(np.max(np.abs(x)))[1] if np.any(x) else 0 for x in X.astype(np.float64)])
    es = np.array([np.frexp(np.max(np.abs(sv)))[1] + 1 if np.any(sv) else 0 for sv in Sv.T])
    ux = np.ldexp(1.0, ex - bits(n) - 1)  # half a unit of x's image, per vector
    us = np.ldexp(1.0, es - bits(k) - 1)  # half a unit of s's image (one binade of slack)
    img = (np.abs(Bd.T) @ (np.abs(Dd) * np.count_nonzero(Ct, axis=1)))[None, :] * ux[:, None] \
        + np.count_nonzero(Bt, axis=0)[None, :] * us[:, None]
    bound = 2 * np.spacing(np.abs(Yo)).astype(np.float64) + 1e-12 * mag + img
    bad = np.abs(Yg.astype(np.float64) - Yo.astype(np.float64)) > bound
    assert not bad.any(), f"{label}: {bad.sum()} outputs differ, worst {np.max(np.abs(Yg - Yo)):.3g}"
    return Yg, Yo


@pytest.mark.parametrize("k,m,n,batch", [(1, 1, 1, 1), (5, 7, 9, 1), (64, 17, 33, 3), (300, 389, 103, 2),
                                         (1000, 16, 2000, 1), (37, 1100, 17, 5),
                                         # x in several LDS chunks of digit operands, rows of C and B
                                         # not a multiple of four words, several component chunks
                                         (600, 5000, 7000, 3), (513, 4100, 6400, 2), (2000, 300, 260, 33)])
def test_random_factors(k, m, n, batch):
    rng = np.random.default_rng(100 + k + m + n)
    Bt, Ct, D = random_factors(rng, k, m, n)
    X = rng.standard_normal((batch, n)).astype(np.float32)
    check(Bt, Ct, D, X, f"k={k} m={m} n={n} batch={batch}")


def test_full_size_attention_shape():
    """k = 7680, 2560 x 2560 (the attention workload's factor shapes), batch 1 and 4."""
    rng = np.random.default_rng(7)
    Bt, Ct, D = random_factors(rng, 7680, 2560, 2560)
    for batch in (1, 4):
        X = rng.standard_normal((batch, 2560)).astype(np.float32)
        check(Bt, Ct, D, X, f"attn batch={batch}")


def test_zero_and_single_vector():
    rng = np.random.default_rng(3)
    Bt, Ct, D = random_factors(rng, 40, 50, 60)
    Z = np.zeros_like(Bt)
    X = rng.standard_normal((2, 60)).astype(np.float32)
    Yg, _ = check(Z, Ct, D, X, "zero B")
    assert np.all(Yg == 0)
    # a 1-D x gives a 1-D y equal to the batched row
    dev = torch.device("cuda:0")
    B = torch.from_numpy(pack(Bt).view(np.int32)).to(dev)
    C = torch.from_numpy(pack(Ct).view(np.int32)).to(dev)
    y1 = erm.apply_factors(B, C, torch.from_numpy(D).to(dev), 50, 60, torch.from_numpy(X[1]).to(dev))
    yb = erm.apply_factors(B, C, torch.from_numpy(D).to(dev), 50, 60, torch.from_numpy(X).to(dev))
    assert np.array_equal(y1.cpu().numpy(), yb[1].cpu().numpy())


def test_factors_of_a_gpu_decomposition():
    """Factors written by externd_decompose feed externd_apply_factors directly; the product
    approximates A x within the decomposition's residual."""
    c = inputs.CONFIGS["lowrank1024"]
    A, _ = inputs.make_input("lowrank1024", m=300, n=260)
    dev = torch.device("cuda:0")
    r = erm.decompose(torch.from_numpy(A).to(dev), 2.0, c["tau"], None, c["als_iters"], 1)
    k = r["k"]
    X = np.random.default_rng(9).standard_normal((3, 260)).astype(np.float32)
    Yg = erm.apply_factors(r["B"], r["C"], r["D"], 300, 260, torch.from_numpy(X).to(dev)).cpu().numpy()
    Bp = r["B"].cpu().numpy().view(np.uint32)
    Cp = r["C"].cpu().numpy().view(np.uint32)
    D = r["D"].cpu().numpy()
    Yo = oracle.apply(Bp, Cp, D, 300, 260, X)
    Bt, Ct = erm.unpack(Bp, 300), erm.unpack(Cp, 260)
    check(Bt, Ct, D, X, "decomposition factors")
    AX = X.astype(np.float64) @ A.T.astype(np.float64)
    resid = np.sqrt(max(0.0, 1.0 - float(r["energy"][-1].item()))) * np.linalg.norm(A.astype(np.float64))
    assert np.all(np.linalg.norm(AX - Yg, axis=1) <= resid * np.linalg.norm(X, axis=1) * (1 + 1e-5) + 1e-4)
    assert np.array_equal(Yg, gpu_apply(Bp, Cp, D, 300, 260, X))  # deterministic
    assert k == erm.rank(300, 260, 2.0)
    del Yo
