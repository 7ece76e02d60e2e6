"""GPU parity of the sequential-deflation path against the oracle (through the C ABI)."""

import json
import os

import numpy as np
import pytest

import oracle
from expanded_rank_matrix_amd import inputs
from tests import _parity as P

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def run_both(A, mu, tau, h, T, block=1):
    g = P.gpu_decompose(A, mu, tau, h, T, block)
    o = oracle.decompose(A, mu, tau, h, T, block)
    return g, o


def test_golden_2x2():
    ex = json.load(open(GOLDEN))["decomposition_2x2"]
    A = np.array(ex["A"], np.float32)
    g = P.gpu_decompose(A, ex["mu"], ex["tau"], None, ex["als_iters"], 1)
    assert oracle.unpack(g["B"], 2).tolist() == ex["u"]
    assert oracle.unpack(g["C"], 2).tolist() == ex["v"]
    assert g["D"].tolist() == ex["d"]
    assert np.allclose(g["energy"], ex["energy"], atol=1e-15, rtol=0)
    assert g["stats"]["fallback_inits"] == ex["fallbacks"]


def test_tiny_oracle_case_every_component():
    c = inputs.CONFIGS["tiny64x48"]
    A, h = inputs.make_input("tiny64x48")
    g, o = run_both(A, c["mu"], c["tau"], h, c["als_iters"])
    f = P.check_free_run(g, o, "tiny64x48", alt=(A, c["mu"], c["tau"], h, c["als_iters"], 1))
    _, mism = P.check_replay(A, c["mu"], c["tau"], h, c["als_iters"], 1, g, np.arange(g["k"]), "tiny64x48")
    assert P.monotone(g["energy"])
    assert f == g["k"] and mism == 0, (f, mism)


@pytest.mark.parametrize("name,m,n", [("lowrank1024", 300, 260), ("attn2560", 333, 257),
                                      ("down2560x9728", 129, 700), ("attn2560", 1, 37),
                                      ("attn2560", 41, 1), ("attn2560", 17, 1100)])
def test_scaled_workloads_free_run_and_replay(name, m, n):
    c = inputs.CONFIGS[name]
    A, h = inputs.make_input(name, m=m, n=n)
    mu = 1.0 if min(m, n) > 1 else 2.0
    g, o = run_both(A, mu, c["tau"], h, 3)
    f = P.check_free_run(g, o, f"{name} {m}x{n}", alt=(A, mu, c["tau"], h, 3, 1))
    k = g["k"]
    sample = sorted(set([0, 1, k // 3, k // 2, k - 1]))
    _, mism = P.check_replay(A, mu, c["tau"], h, 3, 1, g, sample, f"{name} {m}x{n}")
    print(f"{name} {m}x{n}: identical prefix {f} of {k}, replay mismatches {mism}")
    assert P.monotone(g["energy"])


@pytest.mark.parametrize("tau", [0.0, 0.1, 0.5, 1.0])
def test_tau_values(tau):
    A, _ = inputs.make_input("attn2560", m=200, n=150)
    g, o = run_both(A, 0.5, tau, None, 4)
    f = P.check_free_run(g, o, f"tau={tau}", alt=(A, 0.5, tau, None, 4, 1))
    print(f"tau={tau}: identical prefix {f} of {g['k']}")


def test_weighted_sequential():
    A, h = inputs.make_input("down2560x9728", m=150, n=220)
    g, o = run_both(A, 1.0, 0.2, h, 3)
    f = P.check_free_run(g, o, "weighted", alt=(A, 1.0, 0.2, h, 3, 1))
    _, mism = P.check_replay(A, 1.0, 0.2, h, 3, 1, g, [0, 10, 100, g["k"] - 1], "weighted")
    print(f"weighted: identical prefix {f} of {g['k']}, replay mismatches {mism}")


@pytest.mark.parametrize("name,m,n,mu", [("attn2560", 300, 260, 1.0), ("lowrank1024", 1024, 1024, 0.25)])
def test_residual_in_hbm(name, m, n, mu):
    """The unweighted kernel with both residual copies in HBM (residual_hbm): the same factors as
    the oracle and bit-equal to the default LDS-resident run."""
    c = inputs.CONFIGS[name]
    A, h = inputs.make_input(name, m=m, n=n)
    g = P.gpu_decompose(A, mu, c["tau"], h, c["als_iters"], 1, residual_hbm=True)
    assert g["stats"]["residual_lds"] == 0
    o = oracle.decompose(A, mu, c["tau"], h, c["als_iters"], 1)
    f = P.check_free_run(g, o, f"{name} {m}x{n} in HBM", alt=(A, mu, c["tau"], h, c["als_iters"], 1))
    assert f == g["k"], f
    g2 = P.gpu_decompose(A, mu, c["tau"], h, c["als_iters"], 1)
    assert g2["stats"]["residual_lds"] == 1
    for key in ("B", "C", "D", "energy"):
        assert np.array_equal(g[key], g2[key]), key
    # the kernel's bookkeeping (workgroup 0 keeps it in LDS and adds it once at the end) is the
    # same whichever copy of the residual the kernel holds
    for key in ("passes", "early_exits", "fallback_inits", "zero_components", "bytes_algorithmic"):
        assert g["stats"][key] == g2["stats"][key], key


@pytest.mark.parametrize("name,m,n,mu", [("down2560x9728", 120, 9728, 0.5), ("attn2560", 40, 16384, 1.0)])
def test_wide_rows_beyond_the_key_array(name, m, n, mu):
    """Rows so long that the LDS array of fp32 keys no longer fits beside the exchanged vector (and
    the weights): the kernel sizes the key array for the unweighted U-steps only (weighted, 9728
    columns) or drops it (16384 columns) and takes the general selection there.  Same factors as
    the oracle."""
    c = inputs.CONFIGS[name]
    A, h = inputs.make_input(name, m=m, n=n)
    g = P.gpu_decompose(A, mu, c["tau"], h, c["als_iters"], 1)
    o = oracle.decompose(A, mu, c["tau"], h, c["als_iters"], 1)
    f = P.check_free_run(g, o, f"{name} {m}x{n}", alt=(A, mu, c["tau"], h, c["als_iters"], 1))
    assert f == g["k"], f


def test_determinism():
    A, _ = inputs.make_input("lowrank1024", m=512, n=384)
    g1 = P.gpu_decompose(A, 1.5, 0.1, None, 4, 1)
    g2 = P.gpu_decompose(A, 1.5, 0.1, None, 4, 1)
    for key in ("B", "C", "D", "energy"):
        assert np.array_equal(g1[key], g2[key]), key


def test_special_cases():
    # zero matrix
    g = P.gpu_decompose(np.zeros((19, 23), np.float32), 2.0, 0.0, None, 3, 1)
    assert np.all(g["B"] == 0) and np.all(g["C"] == 0) and np.all(g["D"] == 0)
    assert np.all(g["energy"] == 1.0)
    # identity
    n = 40
    g = P.gpu_decompose(np.eye(n, dtype=np.float32), 1.0, 0.0, None, 4, 1)
    assert np.all(oracle.unpack(g["B"][:1], n) == 1) and g["D"][0] == pytest.approx(1.0 / n, rel=1e-7)
    # exact zero residual midway: remaining components are zero, energy 1
    g = P.gpu_decompose(np.array([[1, 2], [3, 4]], np.float32), 3.0, 0.0, None, 4, 1)
    assert np.all(g["D"][3:] == 0) and np.all(g["energy"][2:] == 1.0)
    # 1 x 1
    g = P.gpu_decompose(np.array([[-2.5]], np.float32), 3.0, 0.0, None, 2, 1)
    assert g["D"][0] == 2.5 and oracle.unpack(g["B"], 1)[0, 0] * oracle.unpack(g["C"], 1)[0, 0] == -1
    assert np.all(g["energy"] == 1.0)


def test_error_paths():
    import torch

    import expanded_rank_matrix_amd as erm

    A = torch.zeros((8, 8), dtype=torch.float32, device="cuda")
    A[3, 4] = float("nan")
    with pytest.raises(erm.ExterndError) as e:
        erm.decompose(A, 1.0)
    assert e.value.status == erm.ENONFINITE
    A = torch.ones((8, 8), dtype=torch.float32, device="cuda")
    h = torch.ones(8, dtype=torch.float32, device="cuda")
    h[2] = 0.0
    with pytest.raises(erm.ExterndError) as e:
        erm.decompose(A, 1.0, h=h)
    assert e.value.status == erm.EINVAL
    for kw in (dict(tau=1.5), dict(tau=-0.1), dict(als_iters=0), dict(block=-2)):
        with pytest.raises(erm.ExterndError) as e:
            erm.decompose(A, 1.0, **kw)
        assert e.value.status == erm.EINVAL
    with pytest.raises(erm.ExterndError):
        erm.decompose(A, 0.0)
    # the library still works after errors
    r = erm.decompose(A, 1.0)
    assert r["stats"]["k"] == 8


def test_projection_matches_oracle():
    import torch

    import expanded_rank_matrix_amd as erm

    for L in (1, 5, 48, 64, 511, 512, 513, 1000, 2560, 4099, 9728, 16384):
        X = inputs.random_vectors(1000 + L, 6, L)
        X[1] *= np.float32(1e-3)
        X[2, : L // 2] = 0.0
        X[3] = np.round(X[3] * 2) / 2  # many exact ties
        h = inputs.lognormal_weights(2000 + L, L)
        for tau in (0.0, 0.3, 1.0):
            for hh in (None, h):
                V, PHC = erm.project(torch.from_numpy(X).cuda(), tau,
                                     None if hh is None else torch.from_numpy(hh).cuda())
                V = V.cpu().numpy()
                PHC = PHC.cpu().numpy()
                for r in range(X.shape[0]):
                    v, Po, Ho, So, jo, gap = oracle.project(X[r], tau, hh)
                    if gap > 1e-12:
                        assert np.array_equal(V[r], v), (L, tau, hh is None, r)
                        assert PHC[r, 2] == jo
                        # the reported sums come from the selection's 64-bit fixed point:
                        # each element is truncated by < 2^-47 of max h|x|
                        assert PHC[r, 0] == pytest.approx(Po, rel=1e-9)
                        assert PHC[r, 1] == pytest.approx(Ho, rel=1e-9)


def test_projection_adversarial():
    import torch

    import expanded_rank_matrix_amd as erm

    from tests.test_oracle_projection import ADVERSARIAL

    # flat score (a_i ~ 1/sqrt(i)) forces the refinement / chunked path
    L = 3000
    flat = (1.0 / np.sqrt(np.arange(1, L + 1))).astype(np.float32)
    cases = [np.array(x, np.float32) for x in ADVERSARIAL] + [flat, np.ones(2000, np.float32),
                                                               np.repeat(np.float32([3, 2, 1]), 700)]
    for x in cases:
        for tau in (0.0, 0.5):
            V, PHC = erm.project(torch.from_numpy(x[None, :]).cuda(), tau)
            v, Po, Ho, So, jo, gap = oracle.project(x, tau)
            assert np.array_equal(V.cpu().numpy()[0], v), (x[:8], tau)


def test_matvec_matches_oracle():
    import torch

    import expanded_rank_matrix_amd as erm

    rng = np.random.default_rng(5)
    for m, n in ((1, 1), (37, 53), (256, 2560), (1031, 77)):
        R = rng.standard_normal((m, n)).astype(np.float32)
        u = rng.integers(-1, 2, m).astype(np.int8)
        v = rng.integers(-1, 2, n).astype(np.int8)
        h = inputs.lognormal_weights(3, n)
        Rt = torch.from_numpy(R).cuda()
        w = erm.matvec(Rt, torch.from_numpy(u).cuda(), transpose=True).cpu().numpy()
        z = erm.matvec(Rt, torch.from_numpy(v).cuda(), torch.from_numpy(h).cuda()).cpu().numpy()
        wo = oracle.matvec(R, u, transpose=True)
        zo = oracle.matvec(R, v, h)
        assert np.max(np.abs(w - wo)) <= 1e-12 * max(1.0, np.max(np.abs(wo)))
        assert np.max(np.abs(z - zo)) <= 1e-12 * max(1.0, np.max(np.abs(zo)))
