"""Helpers for GPU-vs-oracle parity checks (test infrastructure).

Contract (numeric conventions of the decomposition engine): ternary factors identical for
every component whose selection gap exceeds 1e-6; scales within 1e-5 relative; matvecs within
1e-5 normwise-relative; energy curve within 1e-4 absolute.  After the first divergence of a
free run (only allowed at a near-tie), later components are compared by replay: the oracle
refits each sampled component from the residual that the GPU's own earlier factors imply.
"""

import numpy as np

import oracle

GAP_TOL = 1e-6
D_RTOL = 1e-5
E_ATOL = 1e-4


def gpu_decompose(A, mu, tau, h, T, block, **options):
    import torch

    import expanded_rank_matrix_amd as erm

    At = torch.from_numpy(np.ascontiguousarray(A)).cuda()
    ht = None if h is None else torch.from_numpy(np.ascontiguousarray(h)).cuda()
    r = erm.decompose(At, mu, tau, ht, T, block, **options)
    torch.cuda.synchronize()
    return dict(B=r["B"].cpu().numpy().view(np.uint32), C=r["C"].cpu().numpy().view(np.uint32),
                D=r["D"].cpu().numpy(), energy=r["energy"].cpu().numpy(), stats=r["stats"], k=r["k"])


def first_divergence(g, o):
    """Index of the first component whose factors differ (len if none)."""
    k = min(g["B"].shape[0], o["B"].shape[0])
    same = (np.all(g["B"][:k] == o["B"][:k], axis=1) & np.all(g["C"][:k] == o["C"][:k], axis=1))
    bad = np.nonzero(~same)[0]
    return int(bad[0]) if len(bad) else k


def check_free_run(g, o, label="", b=1):
    """Identical factors up to the first divergence, which must sit at a near-tie; D and the
    energy curve agree on the common prefix.  Returns the divergence index (for the block path,
    the first component of the first block that differs: the components of a block are fitted
    jointly, so a tie anywhere in the block may change all of them)."""
    k = min(g["B"].shape[0], o["B"].shape[0])
    f = first_divergence(g, o)
    if f < k:
        f = (f // b) * b
        gap = float(np.min(o["gaps"][f:f + b]))
        assert gap <= GAP_TOL, (
            f"{label}: factors diverge at component {f} whose oracle selection gap "
            f"{gap:.3e} exceeds {GAP_TOL}")
    np.testing.assert_allclose(g["D"][:f], o["D"][:f], rtol=D_RTOL, atol=0, err_msg=label)
    assert np.max(np.abs(g["energy"][:f] - o["energy"][:f]), initial=0.0) <= E_ATOL, label
    return f


def check_replay(A, mu, tau, h, T, block, g, sample, label="", upto=0):
    """Refit sampled components (or blocks) from the GPU's own residual history."""
    sample = sorted(set(int(x) for x in sample))
    r = oracle.replay(A, mu, tau, h, T, block, g["B"], g["C"], g["D"], sample, upto=upto)
    b = r["b"]
    mism = 0
    for si, s in enumerate(r["sample"]):
        rows = list(range(s * b, min(s * b + b, g["B"].shape[0]))) if b > 1 else [s]
        slots = [si * b + c for c in range(len(rows))]
        same = [np.array_equal(r["Bo"][sl], g["B"][i]) and np.array_equal(r["Co"][sl], g["C"][i])
                for sl, i in zip(slots, rows)]
        if not all(same):
            # a block is fitted jointly: one near-tie anywhere in it may change every member
            mism += 1
            gap = float(np.min(r["gap_o"][slots]))
            assert gap <= GAP_TOL, (
                f"{label}: component(s) {[i for i, ok in zip(rows, same) if not ok][:8]} differ "
                f"from the oracle refit; smallest gap in the block {gap:.3e}")
            continue
        np.testing.assert_allclose(g["D"][rows], r["Do"][slots], rtol=D_RTOL, atol=0,
                                   err_msg=f"{label}: D[{rows[0]}..]")
    er = r["energy_replay"]
    ok = ~np.isnan(er)
    assert np.max(np.abs(g["energy"][ok] - er[ok]), initial=0.0) <= E_ATOL, label
    return r, mism


def monotone(e):
    return bool(np.all(np.diff(e) >= -1e-12))
