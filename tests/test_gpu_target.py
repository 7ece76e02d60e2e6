"""GPU parity of the energy-target stop and the Prop. 2 safeguard (externd_decompose_ex)
against the oracle, through the C ABI.

Energy target (pith.science, free parameters: mu chosen per matrix to reach a target energy):
targets sit midway between neighbouring values of the oracle's energy curve, so that the stop
index does not hang on the last bits of the energy bookkeeping (the contract for the curve is
1e-4 absolute).  The targeted GPU run must stop at the oracle's index, agree with the oracle's
targeted run on the kept components, and hold the energy over zero components afterwards.

Safeguard (pith.science, major comment 1 on Appendix A's Prop. 2): small random matrices at
mu = 16 drive the residual to the fp32 floor, where the best single entry beats the ALS
component now and then; the GPU's choices and activation count must match the oracle's up to
the first selection near-tie.
"""

import numpy as np
import pytest

import oracle
from expanded_rank_matrix_amd import inputs
from tests import _parity as P

pytestmark = pytest.mark.gpu


def safe_targets(curve, picks, sep=1e-3):
    """Midpoints of the curve at the picked steps whose neighbours are at least sep apart."""
    out = []
    for i in picks:
        lo, hi = float(curve[i - 1]), float(curve[i])
        if hi - lo >= sep:
            out.append((i, 0.5 * (lo + hi)))
    assert out, "no well-separated pick"
    return out


def check_stopped(g, o, used, b=1, label=""):
    k = g["k"]
    assert g["stats"]["components_used"] == used == o["used"], label
    f = P.check_free_run({kk: (v[:used] if hasattr(v, "shape") else v) for kk, v in g.items()},
                         {kk: (v[:used] if hasattr(v, "shape") else v) for kk, v in o.items()},
                         label, b)
    assert f == used, f"{label}: diverged at {f} before the stop at {used}"
    assert np.all(g["B"][used:] == 0) and np.all(g["C"][used:] == 0) and np.all(g["D"][used:] == 0)
    assert np.all(g["energy"][used:] == g["energy"][used - 1]), label
    assert abs(g["stats"]["energy_final_explicit"] - o["energy_explicit"]) <= P.E_ATOL, label
    assert used <= k


@pytest.mark.parametrize("name,m,n,mu,tau,weighted", [
    ("tiny64x48", 64, 48, 2.0, 0.0, False),
    ("attn2560", 300, 260, 1.0, 0.0, False),
    ("down2560x9728", 120, 410, 1.5, 0.0, True),    # weighted (R in HBM)
    ("lowrank1024", 257, 129, 2.0, 0.2, False),
])
def test_sequential_target_stop(name, m, n, mu, tau, weighted):
    A, h = inputs.make_input(name, m=m, n=n)
    if not weighted:
        h = None
    full = oracle.decompose(A, mu, tau, h, 4, 1)
    k = full["k"]
    for i, t in safe_targets(full["energy"], [1, k // 10, k // 3, (2 * k) // 3]):
        g = P.gpu_decompose(A, mu, tau, h, 4, 1, energy_target=t)
        o = oracle.decompose(A, mu, tau, h, 4, 1, energy_target=t)
        assert o["used"] == i + 1
        check_stopped(g, o, i + 1, 1, f"{name} target {t:.6f}")


@pytest.mark.parametrize("block,m,n,mu,weighted", [
    (8, 64, 48, 2.0, False),
    (16, 130, 97, 2.0, True),
    (64, 300, 260, 1.0, False),
    (128, 400, 300, 1.0, False),   # stops in the second 64-component slot of the scale walk
])
def test_block_target_stop_inside_a_block(block, m, n, mu, weighted):
    A, h = inputs.make_input("down2560x9728" if weighted else "attn2560", m=m, n=n)
    if not weighted:
        h = None
    full = oracle.decompose(A, mu, 0.0, h, 3, block)
    k = full["k"]
    picks = [p for p in (block + block // 2, 2 * block - 1, 3 * block, k - 2) if 1 <= p < k]
    for i, t in safe_targets(full["energy"], picks, sep=2e-4):
        g = P.gpu_decompose(A, mu, 0.0, h, 3, block, energy_target=t)
        o = oracle.decompose(A, mu, 0.0, h, 3, block, energy_target=t)
        assert o["used"] == i + 1
        check_stopped(g, o, i + 1, block, f"b={block} target {t:.6f}")


def test_target_edge_cases():
    # target above the final energy: everything is fitted, as without a target
    A, _ = inputs.make_input("tiny64x48")
    for block in (1, 8):
        full = P.gpu_decompose(A, 1.0, 0.0, None, 4, block)
        t = min(1.0, float(full["energy"][-1]) + 1e-3)
        g = P.gpu_decompose(A, 1.0, 0.0, None, 4, block, energy_target=t)
        assert g["stats"]["components_used"] == g["k"]
        for key in ("B", "C", "D", "energy"):
            assert np.array_equal(g[key], full[key]), key
    # zero matrix: the first (zero) component has energy 1 and ends the walk
    for block in (1, 4):
        g = P.gpu_decompose(np.zeros((19, 23), np.float32), 2.0, 0.0, None, 3, block, energy_target=0.3)
        assert g["stats"]["components_used"] == 1
        assert np.all(g["D"] == 0) and np.all(g["energy"] == 1.0) and np.all(g["B"] == 0)
    # residual vanishing midway (2 x 2 example): stop at the first energy-1 component
    A = np.array([[1, 2], [3, 4]], np.float32)
    o = oracle.decompose(A, 3.0, 0.0, None, 4, 1, energy_target=1.0)
    g = P.gpu_decompose(A, 3.0, 0.0, None, 4, 1, energy_target=1.0)
    assert g["stats"]["components_used"] == o["used"]
    assert np.array_equal(g["B"], o["B"]) and np.array_equal(g["D"], o["D"])


@pytest.mark.parametrize("m,n,seed", [(8, 8, 1), (6, 5, 5), (4, 4, 2), (3, 7, 3)])
def test_safeguard_parity_small(m, n, seed):
    A = np.random.default_rng(seed).standard_normal((m, n)).astype(np.float32)
    o = oracle.decompose(A, 16.0, 0.0, None, 4, 1, safeguard=True)
    g = P.gpu_decompose(A, 16.0, 0.0, None, 4, 1, safeguard=True)
    f = P.check_free_run(g, o, f"safeguard {m}x{n}")
    if f == g["k"]:
        assert g["stats"]["safeguard_activations"] == o["counters"][1]
        assert o["counters"][1] > 0  # these cases do exercise the replacement
    else:
        assert f > 0


def test_safeguard_weighted_and_larger():
    # weighted norm (R in HBM) and a multi-workgroup grid: the search spans workgroups
    A, h = inputs.make_input("down2560x9728", m=40, n=300)
    o = oracle.decompose(A, 4.0, 0.0, h, 4, 1, safeguard=True)
    g = P.gpu_decompose(A, 4.0, 0.0, h, 4, 1, safeguard=True)
    f = P.check_free_run(g, o, "safeguard weighted")
    if f == g["k"]:
        assert g["stats"]["safeguard_activations"] == o["counters"][1]
    A, _ = inputs.make_input("attn2560", m=200, n=180)
    o = oracle.decompose(A, 1.0, 0.0, None, 4, 1, safeguard=True)
    g = P.gpu_decompose(A, 1.0, 0.0, None, 4, 1, safeguard=True)
    P.check_free_run(g, o, "safeguard 200x180")
    # without activations the safeguard leaves the result unchanged
    g0 = P.gpu_decompose(A, 1.0, 0.0, None, 4, 1)
    if g["stats"]["safeguard_activations"] == 0:
        for key in ("B", "C", "D", "energy"):
            assert np.array_equal(g[key], g0[key]), key


def test_safeguard_with_target():
    A = np.random.default_rng(5).standard_normal((6, 5)).astype(np.float32)
    full = oracle.decompose(A, 16.0, 0.0, None, 4, 1, safeguard=True)
    for i, t in safe_targets(full["energy"], [3, 10], sep=1e-4):
        o = oracle.decompose(A, 16.0, 0.0, None, 4, 1, safeguard=True, energy_target=t)
        g = P.gpu_decompose(A, 16.0, 0.0, None, 4, 1, safeguard=True, energy_target=t)
        check_stopped(g, o, i + 1, 1, f"safeguard target {t:.6f}")


def test_option_errors():
    import torch

    import expanded_rank_matrix_amd as erm

    A = torch.ones((8, 8), dtype=torch.float32, device="cuda")
    for kw in (dict(energy_target=1.5), dict(energy_target=-0.2), dict(energy_target=float("nan"))):
        with pytest.raises(erm.ExterndError) as e:
            erm.decompose(A, 1.0, **kw)
        assert e.value.status == erm.EINVAL
    with pytest.raises(erm.ExterndError) as e:
        erm.decompose(A, 2.0, block=4, safeguard=True)
    assert e.value.status == erm.EINVAL
