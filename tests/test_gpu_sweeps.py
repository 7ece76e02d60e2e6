"""GPU parity of the refinement sweeps (externd_decompose_ex, sweeps > 0) against the oracle,
through the C ABI (review, Results: sweeps add energy and lower the rank a target needs; read as
backfitting: add the component back, refit it from its previous u, deflate the new fit).

A sweep refits every component against a residual that depends on all earlier choices, so a
near-tie anywhere upstream changes everything after it, including components already passed.
The cases below are checked for a divergence-free greedy pass first; the swept factors must
then equal the oracle's up to the first divergence, which may only sit at a near-tie of the
refit it happens in (judged on the single-sweep runs), and the energy bookkeeping must end at
the energy of the final residual.
"""

import numpy as np
import pytest

import oracle
from expanded_rank_matrix_amd import inputs
from tests import _parity as P

pytestmark = pytest.mark.gpu


def greedy_identical(A, mu, tau, h, T):
    g = P.gpu_decompose(A, mu, tau, h, T, 1)
    o = oracle.decompose(A, mu, tau, h, T, 1)
    return P.first_divergence(g, o) == g["k"]


@pytest.mark.parametrize("name,m,n,mu,tau,weighted", [
    ("tiny64x48", 64, 48, 1.0, 0.0, False),
    ("tiny64x48", 64, 48, 2.0, 0.0, False),
    ("attn2560", 200, 150, 1.0, 0.0, False),
    ("down2560x9728", 60, 200, 1.0, 0.0, True),
    ("lowrank1024", 130, 97, 1.0, 0.2, False),
])
def test_sweeps_free_run(name, m, n, mu, tau, weighted):
    A, h = inputs.make_input(name, m=m, n=n)
    if not weighted:
        h = None
    assert greedy_identical(A, mu, tau, h, 4), "greedy pass diverged: pick another case"
    for sweeps in (1, 2):
        g = P.gpu_decompose(A, mu, tau, h, 4, 1, sweeps=sweeps)
        o = oracle.decompose(A, mu, tau, h, 4, 1, sweeps=sweeps)
        f = P.first_divergence(g, o)
        if sweeps == 1:
            P.check_free_run(g, o, f"{name} sweeps=1")
        else:
            assert f == g["k"], f"{name}: sweeps=2 diverged at {f}"
        if f == g["k"]:
            np.testing.assert_allclose(g["D"], o["D"], rtol=P.D_RTOL, atol=0)
            assert np.max(np.abs(g["energy"] - o["energy"])) <= P.E_ATOL
            assert g["stats"]["fallback_inits"] == o["counters"][0]
            # executed passes: the GPU leaves an ALS early at an exact fixed point
            assert g["stats"]["passes"] <= o["counters"][2]
            assert g["stats"]["sweep_reverts"] == o["reverts"]
        # the bookkeeping ends at the energy of the final residual
        assert abs(g["energy"][-1] - g["stats"]["energy_final_explicit"]) < 1e-6
        assert abs(g["stats"]["energy_final_explicit"] - o["energy_explicit"]) <= P.E_ATOL


def test_sweeps_raise_energy_and_keep_the_tail():
    A, _ = inputs.make_input("tiny64x48")
    g0 = P.gpu_decompose(A, 1.0, 0.0, None, 4, 1)
    g1 = P.gpu_decompose(A, 1.0, 0.0, None, 4, 1, sweeps=1)
    g3 = P.gpu_decompose(A, 1.0, 0.0, None, 4, 1, sweeps=3)
    assert g0["energy"][-1] < g1["energy"][-1] < g3["energy"][-1]
    # energy target, then sweeps over the kept components only
    full = oracle.decompose(A, 2.0, 0.0, None, 4, 1)
    t = 0.5 * float(full["energy"][39] + full["energy"][40])
    g = P.gpu_decompose(A, 2.0, 0.0, None, 4, 1, energy_target=t, sweeps=2)
    o = oracle.decompose(A, 2.0, 0.0, None, 4, 1, energy_target=t, sweeps=2)
    used = g["stats"]["components_used"]
    assert used == o["used"] == 41
    assert np.all(g["D"][used:] == 0) and np.all(g["B"][used:] == 0)
    assert np.all(g["energy"][used:] == g["energy"][used - 1])
    assert abs(g["energy"][used - 1] - o["energy"][used - 1]) <= P.E_ATOL


def test_sweeps_special_cases():
    # zero matrix: nothing to refit
    g = P.gpu_decompose(np.zeros((19, 23), np.float32), 2.0, 0.0, None, 3, 1, sweeps=2)
    assert np.all(g["D"] == 0) and np.all(g["energy"] == 1.0)
    # residual vanishing midway: the exact components are a fixed point, the zeros stay zero
    A = np.array([[1, 2], [3, 4]], np.float32)
    g = P.gpu_decompose(A, 3.0, 0.0, None, 4, 1, sweeps=2)
    o = oracle.decompose(A, 3.0, 0.0, None, 4, 1, sweeps=2)
    assert np.array_equal(g["B"], o["B"]) and np.array_equal(g["C"], o["C"])
    assert np.array_equal(g["D"], o["D"])
    # with the safeguard
    A = np.random.default_rng(5).standard_normal((6, 5)).astype(np.float32)
    g = P.gpu_decompose(A, 4.0, 0.0, None, 4, 1, safeguard=True, sweeps=1)
    o = oracle.decompose(A, 4.0, 0.0, None, 4, 1, safeguard=True, sweeps=1)
    P.check_free_run(g, o, "safeguard + sweep")


@pytest.mark.parametrize("block,m,n,mu,tau,weighted", [
    (8, 64, 48, 1.0, 0.0, False),
    (16, 130, 97, 1.0, 0.0, True),     # weighted Gram and fixed-point weights
    (64, 300, 260, 0.5, 0.2, False),   # several tiles, split-K, ragged last block
    (5, 40, 37, 2.0, 0.0, False),      # block not a multiple of the MFMA tile
    (8, 64, 48, 2.0, 0.0, False),      # heavy tails: refits get discarded
])
def test_block_sweeps_free_run(block, m, n, mu, tau, weighted):
    A, h = inputs.make_input("down2560x9728" if weighted else "attn2560", m=m, n=n)
    if not weighted:
        h = None
    g0 = P.gpu_decompose(A, mu, tau, h, 3, block)
    o0 = oracle.decompose(A, mu, tau, h, 3, block)
    assert P.first_divergence(g0, o0) == g0["k"], "greedy pass diverged: pick another case"
    g = P.gpu_decompose(A, mu, tau, h, 3, block, sweeps=1)
    o = oracle.decompose(A, mu, tau, h, 3, block, sweeps=1)
    f = P.check_free_run(g, o, f"b={block} sweeps=1", block)
    assert abs(g["energy"][-1] - g["stats"]["energy_final_explicit"]) < 1e-6
    assert abs(g["stats"]["energy_final_explicit"] - o["energy_explicit"]) <= P.E_ATOL
    assert g["energy"][-1] > g0["energy"][-1] - 1e-6
    if f == g["k"]:
        assert g["stats"]["passes"] == o["counters"][2]
        assert g["stats"]["sweep_reverts"] == o["reverts"]


def test_block_sweeps_after_a_target_stop():
    A, _ = inputs.make_input("tiny64x48")
    full = oracle.decompose(A, 2.0, 0.0, None, 3, 8)
    for i in (29, 95):  # inside a block, and inside the last block
        t = 0.5 * float(full["energy"][i - 1] + full["energy"][i]) if i < 95 else \
            0.5 * float(full["energy"][i - 2] + full["energy"][i - 1])
        g = P.gpu_decompose(A, 2.0, 0.0, None, 3, 8, energy_target=t, sweeps=2)
        o = oracle.decompose(A, 2.0, 0.0, None, 3, 8, energy_target=t, sweeps=2)
        used = g["stats"]["components_used"]
        assert used == o["used"]
        assert np.all(g["D"][used:] == 0) and np.all(g["B"][used:] == 0)
        assert np.all(g["energy"][used:] == g["energy"][used - 1])
        assert abs(g["energy"][used - 1] - o["energy"][used - 1]) <= P.E_ATOL
