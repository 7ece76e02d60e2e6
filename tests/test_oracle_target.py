"""Pins of the oracle's energy-target stop (pith.science free parameters: mu is the accuracy
dial, chosen per matrix to reach a target energy).

The stop is defined from the untargeted energy curve: the greedy components do not depend on k,
so the targeted run must be the untargeted run cut after the first component whose energy
reaches the target.  Checked here against that definition, computed in numpy from the full
curve, and against an explicit residual rebuilt in numpy from the emitted factors (which shows
that dropped block components were not applied):
* used = 1 + the smallest i with energy[i] >= target (a target equal to a curve value stops
  exactly there, so a strict comparison fails);
* the first `used` components and energies equal the untargeted run's; later components are
  zero with the last energy held;
* the explicit final energy equals 1 - |A - sum_{i < used} d_i u_i v_i^T|_H^2 / |A|_H^2;
* a target above the final energy changes nothing; the zero matrix and a residual that
  vanishes midway stop at their first energy-1 component.
"""

import numpy as np
import pytest

import oracle
from expanded_rank_matrix_amd import inputs


def unpacked(r, m, n):
    return oracle.unpack(r["B"], m), oracle.unpack(r["C"], n), r["D"]


def explicit_energy(A, U, V, D, used, h=None):
    A64 = A.astype(np.float64)
    R = A64 - (U[:used].T.astype(np.float64) * D[:used].astype(np.float64)) @ V[:used].astype(np.float64)
    hh = np.ones(A.shape[1]) if h is None else h.astype(np.float64)
    return 1.0 - np.sum(R * R * hh) / np.sum(A64 * A64 * hh)


def expected_used(curve, target):
    hit = np.nonzero(curve >= target)[0]
    return int(hit[0]) + 1 if hit.size else len(curve)


def check_cut(A, full, cut, target, h=None):
    m, n = A.shape
    used = expected_used(full["energy"], target)
    assert cut["used"] == used
    k = full["k"]
    assert np.array_equal(cut["B"][:used], full["B"][:used])
    assert np.array_equal(cut["C"][:used], full["C"][:used])
    assert np.array_equal(cut["D"][:used], full["D"][:used])
    assert np.array_equal(cut["energy"][:used], full["energy"][:used])
    assert np.all(cut["B"][used:] == 0) and np.all(cut["C"][used:] == 0)
    assert np.all(cut["D"][used:] == 0)
    assert np.all(cut["energy"][used:] == cut["energy"][used - 1])
    assert np.all(np.isinf(cut["gaps"][used:]))
    assert cut["energy"][used - 1] >= target or used == k
    if used > 1:
        assert cut["energy"][used - 2] < target
    U, V, D = unpacked(cut, m, n)
    assert abs(cut["energy_explicit"] - explicit_energy(A, U, V, D, used, h)) < 2e-6
    return used


def targets_from(curve, picks):
    """Targets at exact curve values and midway between neighbours."""
    out = []
    for i in picks:
        out.append(float(curve[i]))
        out.append(0.5 * float(curve[i - 1] + curve[i]))
    return out


@pytest.mark.parametrize("case", ["plain", "weighted", "tau"])
def test_sequential_stop_is_the_cut_curve(case):
    A, h = inputs.make_input("tiny64x48")
    hh = h if case == "weighted" else None
    tau = 0.3 if case == "tau" else 0.0
    full = oracle.decompose(A, 2.0, tau, hh, 4, 1)
    for t in targets_from(full["energy"], [1, 7, 40, 95]):
        cut = oracle.decompose(A, 2.0, tau, hh, 4, 1, energy_target=t)
        check_cut(A, full, cut, t, hh)


@pytest.mark.parametrize("b", [4, 8])
def test_block_stop_inside_a_block(b):
    A, _ = inputs.make_input("tiny64x48")
    full = oracle.decompose(A, 2.0, 0.0, None, 3, b)
    curve = full["energy"]
    # stops at a block's first, a middle and its last component
    picks = [b, b + b // 2 - 1, 2 * b - 1, 5 * b + 2]
    for t in targets_from(curve, picks):
        cut = oracle.decompose(A, 2.0, 0.0, None, 3, b, energy_target=t)
        used = check_cut(A, full, cut, t)
        assert 1 <= used <= full["k"]


def test_target_above_final_energy_changes_nothing():
    A, _ = inputs.make_input("tiny64x48")
    for b in (1, 8):
        full = oracle.decompose(A, 1.0, 0.0, None, 4, b)
        t = min(1.0, float(full["energy"][-1]) + 1e-3)
        cut = oracle.decompose(A, 1.0, 0.0, None, 4, b, energy_target=t)
        assert cut["used"] == full["k"]
        for key in ("B", "C", "D", "energy"):
            assert np.array_equal(cut[key], full[key])


def test_zero_and_vanishing_residual_stop_at_energy_one():
    Z = np.zeros((19, 23), np.float32)
    for b in (1, 4):
        r = oracle.decompose(Z, 2.0, 0.0, None, 3, b, energy_target=0.5)
        assert r["used"] == 1
        assert np.all(r["D"] == 0) and np.all(r["energy"] == 1.0)
    # the hand-worked 2x2 reaches R == 0 after three components (energy 1 from there on)
    A = np.array([[1, 2], [3, 4]], np.float32)
    full = oracle.decompose(A, 3.0, 0.0, None, 4, 1)
    first_one = int(np.nonzero(full["energy"] == 1.0)[0][0])
    cut = oracle.decompose(A, 3.0, 0.0, None, 4, 1, energy_target=1.0)
    assert cut["used"] == first_one + 1
    assert cut["counters"][3] == 0  # no zero component was fitted before the stop


def test_target_with_safeguard():
    rng = np.random.default_rng(5)
    A = rng.standard_normal((6, 5)).astype(np.float32)
    full = oracle.decompose(A, 16.0, 0.0, None, 4, 1, safeguard=True)
    for t in targets_from(full["energy"], [3, 20, 50]):
        cut = oracle.decompose(A, 16.0, 0.0, None, 4, 1, safeguard=True, energy_target=t)
        check_cut(A, full, cut, t)
