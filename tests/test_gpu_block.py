"""GPU parity of the block-ALS path (block size b >= 2) against the oracle (through the C ABI).

The components of a block are fitted jointly (Eq. 3 target with the Gram solves), so parity is
judged per block: a block either matches the oracle exactly or holds a selection near-tie.
"""

import numpy as np
import pytest

import oracle
from expanded_rank_matrix_amd import inputs
from tests import _parity as P

pytestmark = pytest.mark.gpu


def run_both(A, mu, tau, h, T, block, k_limit=0):
    g = P.gpu_decompose(A, mu, tau, h, T, block)
    o = oracle.decompose(A, mu, tau, h, T, block, k_limit=k_limit)
    return g, o


def blocks_of(g, A, block):
    m, n = A.shape
    b = oracle.resolve_block(block, m, n, g["k"])
    return b, -(-g["k"] // b)


@pytest.mark.parametrize("block", [2, 4, 16, 48])
def test_tiny_blocks_every_component(block):
    c = inputs.CONFIGS["tiny64x48"]
    A, h = inputs.make_input("tiny64x48")
    g, o = run_both(A, c["mu"], c["tau"], h, 2, block)
    b, nb = blocks_of(g, A, block)
    f = P.check_free_run(g, o, f"tiny b={block}", b, alt=(A, c["mu"], c["tau"], h, 2, block))
    _, mism = P.check_replay(A, c["mu"], c["tau"], h, 2, block, g, np.arange(nb), f"tiny b={block}")
    print(f"tiny b={block}: identical prefix {f} of {g['k']}, replay mismatches {mism} of {nb} blocks")
    assert f >= b
    assert P.monotone(g["energy"])
    if f == g["k"]:
        assert g["stats"]["passes"] == o["counters"][2]
        assert g["stats"]["fallback_inits"] == o["counters"][0]
        assert g["stats"]["block"] == b


@pytest.mark.parametrize("name,m,n,mu,block", [
    ("mlp9728x2560", 389, 103, 2.0, 16),     # ragged last block (206 = 12 x 16 + 14)
    ("down2560x9728", 103, 389, 3.0, 32),    # weighted, 309 = 9 x 32 + 21
    ("attn2560", 700, 650, 0.5, 64),         # several 64-tiles with ragged tails, split-K
    ("lowrank1024", 300, 260, 1.0, -1),      # default block size min(256, min(m, n) / 8)
    ("attn2560", 300, 280, 1.0, 256),        # largest block
    ("attn2560", 333, 257, 1.0, 100),        # block not a multiple of the MFMA tile
    ("attn2560", 400, 360, 1.0, 160),        # three components per lane in the scale walk
    ("attn2560", 1, 37, 2.0, 2),
    ("attn2560", 41, 1, 2.0, 2),
    ("attn2560", 17, 1100, 1.0, 8),
])
def test_scaled_blocks_free_run_and_replay(name, m, n, mu, block):
    c = inputs.CONFIGS[name]
    A, h = inputs.make_input(name, m=m, n=n)
    tau = c["tau"]
    g, o = run_both(A, mu, tau, h, 3, block)
    b, nb = blocks_of(g, A, block)
    label = f"{name} {m}x{n} b={b}"
    f = P.check_free_run(g, o, label, b, alt=(A, mu, tau, h, 3, block))
    _, mism = P.check_replay(A, mu, tau, h, 3, block, g, sorted({0, 1 % nb, nb // 2, nb - 1}), label)
    print(f"{label}: identical prefix {f} of {g['k']}, replay mismatches {mism}")
    assert P.monotone(g["energy"]), label


def test_update_wide_scale_range():
    """Two entries ~3e6 times the noise: the first block's scales span more than 2^26, so some
    are not multiples of 2^(E - 45) (max |d| < 2^E) and the residual update cannot take its int8
    path; it sums in fp64 instead.  The next blocks, which see that update, still match the
    oracle.  (Noise far smaller still would fall below the contractions' fixed-point grid, which
    is relative to max |R|, and cost the small scales their last digits.)"""
    rng = np.random.default_rng(7)
    m, n, b = 96, 80, 8
    A = (rng.standard_normal((m, n)) * 1e-2).astype(np.float32)
    A[3, 5] = 3.0e4
    A[10, 40] = -2.0e4
    g, o = run_both(A, 0.5, 0.3, None, 2, b)
    d0 = np.abs(g["D"][:b].astype(np.float64))
    d0 = d0[d0 > 0]
    e = np.frexp(d0.max())[1]
    off_grid = int(np.sum(np.ldexp(d0, 45 - e) != np.rint(np.ldexp(d0, 45 - e))))
    assert off_grid > 0, "the block's scales must defeat the fixed-point grid of the update"
    f = P.check_free_run(g, o, "wide-range", b, alt=(A, 0.5, 0.3, None, 2, b))
    print(f"wide-range: identical prefix {f} of {g['k']}, d span {d0.max() / d0.min():.3e}, "
          f"{off_grid} scales off the grid")
    assert f >= 2 * b


def test_block_determinism():
    A, h = inputs.make_input("down2560x9728", m=512, n=700)
    g1 = P.gpu_decompose(A, 1.0, 0.2, h, 3, 32)
    g2 = P.gpu_decompose(A, 1.0, 0.2, h, 3, 32)
    for key in ("B", "C", "D", "energy"):
        assert np.array_equal(g1[key], g2[key]), key


@pytest.mark.parametrize("m,n,block", [(160, 6200, 32), (200, 6200, 128)])
def test_split_gram_long_rows(m, n, block):
    """Weighted Gram over rows longer than 3072 (split over K, partials added by the last
    workgroup of each tile) and the inverse inside the contraction launch: two runs agree bit for
    bit, and the run agrees with the oracle over the first blocks and on a replayed block."""
    A, h = inputs.make_input("down2560x9728", m=m, n=n)
    g1 = P.gpu_decompose(A, 0.5, 0.2, h, 2, block)
    g2 = P.gpu_decompose(A, 0.5, 0.2, h, 2, block)
    for key in ("B", "C", "D", "energy"):
        assert np.array_equal(g1[key], g2[key]), key
    o = oracle.decompose(A, 0.5, 0.2, h, 2, block, k_limit=2 * block)
    label = f"split gram {m}x{n} b={block}"
    f = P.check_free_run(g1, o, label, block, alt=(A, 0.5, 0.2, h, 2, block))
    nb = -(-g1["k"] // block)
    _, mism = P.check_replay(A, 0.5, 0.2, h, 2, block, g1, [0, nb - 1], label)
    print(f"{label}: identical prefix {f} of {g1['k']}, replay mismatches {mism}")


def test_block_integer_inputs_exact():
    """Small integer matrices: every fp64 sum is exact in any order, so the GPU must reproduce
    the oracle bit for bit, ties included."""
    rng = np.random.default_rng(11)
    for (m, n, mu, block) in [(2, 2, 3.0, 2), (6, 5, 2.0, 3), (12, 9, 1.0, 4), (9, 12, 2.0, 5)]:
        A = rng.integers(-3, 4, size=(m, n)).astype(np.float32)
        g, o = run_both(A, mu, 0.0, None, 3, block)
        assert np.array_equal(g["B"], o["B"]) and np.array_equal(g["C"], o["C"]), (m, n, block)
        assert np.array_equal(g["D"], o["D"]), (m, n, block)
        np.testing.assert_allclose(g["energy"], o["energy"], rtol=0, atol=1e-12)


def test_block_special_cases():
    # zero matrix
    g = P.gpu_decompose(np.zeros((19, 23), np.float32), 2.0, 0.0, None, 3, 4)
    assert np.all(g["B"] == 0) and np.all(g["C"] == 0) and np.all(g["D"] == 0)
    assert np.all(g["energy"] == 1.0)
    # identity: compare with the oracle exactly (integer data)
    n = 40
    A = np.eye(n, dtype=np.float32)
    g, o = run_both(A, 1.0, 0.0, None, 4, 8)
    assert np.array_equal(g["B"], o["B"]) and np.array_equal(g["C"], o["C"])
    assert np.array_equal(g["D"], o["D"])
    # rank-one ternary matrix: the first component recovers it and the rest are zero
    rng = np.random.default_rng(3)
    u = rng.choice([-1, 0, 1], size=30).astype(np.float32)
    v = rng.choice([-1, 0, 1], size=20).astype(np.float32)
    u[0] = v[0] = 1
    A = 0.75 * np.outer(u, v)
    g, o = run_both(A, 1.0, 0.0, None, 3, 4)
    assert np.array_equal(g["B"], o["B"]) and np.array_equal(g["D"], o["D"])
    assert g["energy"][-1] == pytest.approx(1.0, abs=1e-12)
    # block larger than k is clamped to k
    A, _ = inputs.make_input("attn2560", m=20, n=30)
    g = P.gpu_decompose(A, 0.5, 0.0, None, 2, 64)
    assert g["stats"]["block"] == g["k"] == 10
