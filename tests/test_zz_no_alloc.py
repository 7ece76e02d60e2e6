"""The allocation-free inference entry point (externd_apply_factors_static, a fixed per-GPU
workspace inside the library) against externd_apply_factors on the same inputs: bit-equal
outputs on two calls in a row, the second smaller; oversize requests are rejected."""

import numpy as np
import pytest

from expanded_rank_matrix_amd import inputs
from tests import _parity as P

pytestmark = pytest.mark.gpu


def _factors(name, m, n, mu):
    c = inputs.CONFIGS[name]
    A, h = inputs.make_input(name, m=m, n=n)
    return P.gpu_decompose(A, mu, c["tau"], h, c["als_iters"], 1)


def test_static_workspace_matches_allocating_entry_point():
    import torch

    import expanded_rank_matrix_amd as erm

    cases = [("attn2560", 700, 650, 1.5, 7, 11), ("lowrank1024", 300, 260, 1.0, 1, 3)]
    for (name, m, n, mu, batch, seed) in cases:  # the second call is smaller in every size
        g = _factors(name, m, n, mu)
        B = torch.from_numpy(g["B"].view(np.int32)).cuda()
        C = torch.from_numpy(g["C"].view(np.int32)).cuda()
        D = torch.from_numpy(g["D"]).cuda()
        X = torch.from_numpy(inputs.random_vectors(seed, batch, n)).cuda()
        ref = erm.apply_factors(B, C, D, m, n, X)
        Y = torch.full((batch, m), float("nan"), dtype=torch.float32, device="cuda")
        erm.apply_factors_static(B, C, D, m, n, X, out=Y)
        torch.cuda.synchronize()
        assert torch.equal(Y, ref), (name, batch)
    # a request beyond the fixed workspace is refused before any work
    k, m, n = 7680, 2560, 2560
    B = torch.zeros((k, erm.packed_words(m)), dtype=torch.int32, device="cuda")
    C = torch.zeros((k, erm.packed_words(n)), dtype=torch.int32, device="cuda")
    D = torch.zeros(k, dtype=torch.float32, device="cuda")
    X = torch.zeros((300, n), dtype=torch.float32, device="cuda")
    with pytest.raises(erm.ExterndError) as e:
        erm.apply_factors_static(B, C, D, m, n, X)
    assert e.value.status == erm.EINVAL
