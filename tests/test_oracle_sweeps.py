"""Pins of the oracle's refinement sweeps (review, Results: sweeps add energy and lower the rank
a target needs; the reading is backfitting: add a component's contribution back, refit it from
its previous u, deflate the new fit).

Checked against what the mathematics fixes, not against the oracle's formulas:
* the energy bookkeeping through the add-backs ends at the explicit energy of the emitted
  factors, 1 - |A - sum_i d_i u_i v_i^T|_H^2 / |A|_H^2, rebuilt here in numpy (a wrong sign or
  a dropped term of the add-back energy breaks it), on both engines, weighted and with tau;
* with tau = 0 and uniform weights every refit removes at least what the old component removed
  (the warm-started V-step is the exact optimum for the old u, and the scale is optimal), so the
  energy never falls within a sweep or from one sweep to the next;
* an exact ternary rank-one matrix is a fixed point: sweeps change nothing;
* the block engine at b = 1 gives the sequential engine's sweeps (the projection is invariant
  to the positive scale (u^T u + eps)^-1);
* with an energy target, components after the stop stay zero and hold the final energy;
* a refit that would leave more residual than the old component (block) is discarded, so no
  sweep lowers the energy by more than the 1e-9 |A|^2 margin per refit; on a heavy-tailed input
  the block refits do get discarded, and the bookkeeping still matches the explicit energy.
"""

import numpy as np
import pytest

import oracle
from expanded_rank_matrix_amd import inputs


def explicit_energy(A, r, h=None):
    m, n = A.shape
    U = oracle.unpack(r["B"], m).astype(np.float64)
    V = oracle.unpack(r["C"], n).astype(np.float64)
    A64 = A.astype(np.float64)
    R = A64 - (U.T * r["D"].astype(np.float64)) @ V
    hh = np.ones(n) if h is None else h.astype(np.float64)
    return 1.0 - np.sum(R * R * hh) / np.sum(A64 * A64 * hh)


@pytest.mark.parametrize("block,weighted,tau", [(1, False, 0.0), (1, True, 0.0), (1, False, 0.3),
                                                (8, False, 0.0), (8, True, 0.2), (5, False, 0.0)])
def test_bookkeeping_matches_explicit_energy(block, weighted, tau):
    A, h = inputs.make_input("down2560x9728", m=48, n=64)
    if not weighted:
        h = None
    for sweeps in (1, 3):
        r = oracle.decompose(A, 1.0, tau, h, 3, block, sweeps=sweeps)
        ex = explicit_energy(A, r, h)
        assert abs(r["energy"][-1] - ex) < 1e-7
        assert abs(r["energy_explicit"] - ex) < 1e-7


def test_energy_never_falls_tau0_uniform():
    A, _ = inputs.make_input("tiny64x48")
    prev = oracle.decompose(A, 1.0, 0.0, None, 4, 1)["energy"][-1]
    for sweeps in (1, 2, 3):
        r = oracle.decompose(A, 1.0, 0.0, None, 4, 1, sweeps=sweeps)
        e = r["energy"]
        assert np.all(np.diff(e) >= -1e-9)   # within the last sweep
        assert e[0] >= prev - 1e-9           # across sweeps
        assert e[-1] > prev                  # and the sweep does add energy here
        prev = e[-1]


def test_exact_rank_one_is_a_fixed_point():
    rng = np.random.default_rng(3)
    u = rng.integers(-1, 2, 23).astype(np.float32)
    v = rng.integers(-1, 2, 17).astype(np.float32)
    u[0], v[0] = 1, 1
    A = 0.75 * np.outer(u, v).astype(np.float32)
    for block in (1, 4):
        r0 = oracle.decompose(A, 1.0, 0.0, None, 4, block)
        r2 = oracle.decompose(A, 1.0, 0.0, None, 4, block, sweeps=2)
        for key in ("B", "C", "D"):
            assert np.array_equal(r0[key], r2[key]), key
        assert r2["energy"][-1] == pytest.approx(1.0, abs=1e-12)


def test_block_engine_b1_equals_sequential_sweeps():
    for m, n, seed in [(20, 16, 1), (64, 48, 0)]:
        A = np.random.default_rng(seed).standard_normal((m, n)).astype(np.float32)
        rs = oracle.decompose(A, 1.0, 0.0, None, 4, 1, sweeps=2)
        rb = oracle.decompose(A, 1.0, 0.0, None, 4, 1, sweeps=2, block_engine=True)
        for key in ("B", "C", "D"):
            assert np.array_equal(rs[key], rb[key]), key
        assert np.allclose(rs["energy"], rb["energy"], atol=1e-12)


@pytest.mark.parametrize("block", [1, 8])
def test_sweeps_after_a_target_stop(block):
    A, _ = inputs.make_input("tiny64x48")
    full = oracle.decompose(A, 2.0, 0.0, None, 3, block)
    t = 0.5 * float(full["energy"][29] + full["energy"][30])
    r = oracle.decompose(A, 2.0, 0.0, None, 3, block, energy_target=t, sweeps=2)
    used = r["used"]
    assert used == 31
    assert np.all(r["D"][used:] == 0) and np.all(r["B"][used:] == 0)
    assert np.all(r["energy"][used:] == r["energy"][used - 1])
    assert abs(r["energy"][used - 1] - explicit_energy(A, r)) < 1e-7
    assert r["energy"][used - 1] > full["energy"][used - 1] - 1e-9


def test_zero_matrix_with_sweeps():
    r = oracle.decompose(np.zeros((9, 7), np.float32), 2.0, 0.0, None, 3, 1, sweeps=2)
    assert np.all(r["D"] == 0) and np.all(r["energy"] == 1.0)


@pytest.mark.parametrize("block", [1, 8])
def test_discarded_refits_keep_energy(block):
    A, _ = inputs.make_input("attn2560", m=64, n=48)   # heavy tails and outlier columns
    prev = oracle.decompose(A, 1.0, 0.0, None, 3, block)
    for sweeps in (1, 2):
        r = oracle.decompose(A, 1.0, 0.0, None, 3, block, sweeps=sweeps)
        nref = sweeps * (-(-r["k"] // block))
        assert r["energy"][-1] >= prev["energy"][-1] - 1e-9 * nref
        assert abs(r["energy"][-1] - explicit_energy(A, r)) < 1e-7
        prev = r
    if block > 1:
        assert r["reverts"] > 0
