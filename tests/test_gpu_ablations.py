"""GPU parity of the ablation switches (externd_options.ablation) against the oracle, through the
C ABI (review, Validation: the pages' ablations; pith.science, Sec. 2.3: decorrelated block
targets).  Bit 1: the block path's batched targets without Eq. 3's decorrelation; bit 2: the
V-step projection without the importance weights (both paths).  Joint fitting is the block path
with one block of all k components.
"""

import numpy as np
import pytest

import oracle
from expanded_rank_matrix_amd import inputs
from tests import _parity as P

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,m,n,mu,block,ablation", [
    ("tiny64x48", 64, 48, 1.0, 8, 1),
    ("mlp9728x2560", 300, 130, 1.0, 64, 1),
    ("down2560x9728", 64, 160, 1.0, 8, 2),
    ("down2560x9728", 96, 200, 1.0, 16, 3),
    ("down2560x9728", 64, 160, 1.0, 1, 2),      # sequential path, unweighted V-step projection
    ("down2560x9728", 120, 410, 0.5, 1, 2),
])
def test_ablation_parity(name, m, n, mu, block, ablation):
    A, h = inputs.make_input(name, m=m, n=n)
    g = P.gpu_decompose(A, mu, 0.0, h, 3, block, ablation=ablation)
    o = oracle.decompose(A, mu, 0.0, h, 3, block, ablation=ablation)
    b = oracle.resolve_block(block, m, n, g["k"])
    f = P.check_free_run(g, o, f"{name} b={block} ablation={ablation}", b)
    assert f >= min(g["k"], 2 * b)
    if f == g["k"]:
        assert abs(g["stats"]["energy_final_explicit"] - o["energy_explicit"]) <= P.E_ATOL


def test_joint_fitting_collapses_on_the_gpu():
    A, _ = inputs.make_input("tiny64x48")
    seq = P.gpu_decompose(A, 2.0, 0.0, None, 4, 1)
    k = seq["k"]
    joint = P.gpu_decompose(A, 2.0, 0.0, None, 4, k)
    o = oracle.decompose(A, 2.0, 0.0, None, 4, k)
    P.check_free_run(joint, o, "joint", k)
    assert joint["energy"][-1] < seq["energy"][-1] - 0.1
