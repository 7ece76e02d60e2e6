"""Helpers for GPU-vs-oracle parity checks (test infrastructure).

Contract (numeric conventions of the decomposition engine): ternary factors identical for
every component whose selection gap exceeds 1e-6; scales within 1e-5 relative; matvecs within
1e-5 normwise-relative; energy curve within 1e-4 absolute.

A difference is excused only when it is an equally good alternative, not merely because some
selection was close: the first differing component (block) of a free run, and every differing
refit of a replay, must sit at a selection gap <= 1e-6 AND the GPU's component (block) must
remove, from the same replayed residual, at least (1 - 1e-6) of the energy that the oracle's own
refit removes (the component's decrease 2 d p - d^2 q; for a block, the sum over its energy walk).
After the first divergence of a free run later components are compared by replay: the oracle
refits each sampled component (block) from the residual that the GPU's own earlier factors imply.
"""

import hashlib
import os

import numpy as np

import oracle

GAP_TOL = 1e-6
D_RTOL = 1e-5
E_ATOL = 1e-4
ALT_RTOL = 1e-6   # an excused divergence removes at least (1 - ALT_RTOL) of the oracle refit's decrease

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


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
    """Index of the first component whose ternary factors differ (len if none)."""
    k = min(g["B"].shape[0], o["B"].shape[0])
    same = (np.all(g["B"][:k] == o["B"][:k], axis=1) & np.all(g["C"][:k] == o["C"][:k], axis=1))
    bad = np.nonzero(~same)[0]
    return int(bad[0]) if len(bad) else k


def check_alternative(A, mu, tau, h, T, block, g, s, label="", r=None):
    """The GPU's component (block) s against the oracle's refit of it from the same replayed
    residual: the GPU's must remove at least (1 - ALT_RTOL) of what the refit removes.  Returns
    (gpu decrease, oracle decrease) in units of |A|^2_H."""
    if r is None:
        m, n = A.shape
        b = oracle.resolve_block(block, m, n, g["k"])
        r = oracle.replay(A, mu, tau, h, T, block, g["B"], g["C"], g["D"], [s],
                          upto=min(g["k"], (s + 1) * b))
    b = r["b"]
    si = int(np.nonzero(r["sample"] == s)[0][0])
    c0, c1 = s * b, min(s * b + b, g["B"].shape[0])
    er = r["energy_replay"]
    before = er[c0 - 1] if c0 > 0 else 0.0
    dec_g = float(er[c1 - 1] - before)
    dec_o = float(np.sum(r["dec_o"][si * b: si * b + (c1 - c0)]))
    assert dec_g >= dec_o - ALT_RTOL * abs(dec_o) - 1e-15, (
        f"{label}: component(s) {c0}..{c1 - 1} differ from the oracle's refit and remove less "
        f"energy ({dec_g:.12e} against {dec_o:.12e}): not an equally good alternative")
    return dec_g, dec_o


def check_free_run(g, o, label="", b=1, alt=None):
    """Identical factors up to the first divergence, which must sit at a near-tie (and, when
    ``alt`` = (A, mu, tau, h, T, block) is given, be an equally good alternative on the replayed
    residual); D and the energy curve agree on the common prefix.  Returns the divergence index
    (for the block path, the first component of the first block that differs: the components of
    a block are fitted jointly, so a tie anywhere in the block may change all of them)."""
    k = min(g["B"].shape[0], o["B"].shape[0])
    f = first_divergence(g, o)
    if f < k:
        f = (f // b) * b
        gap = float(np.min(o["gaps"][f:f + b]))
        assert gap <= GAP_TOL, (
            f"{label}: factors diverge at component {f} whose oracle selection gap "
            f"{gap:.3e} exceeds {GAP_TOL}")
        if alt is not None:
            check_alternative(*alt, g, f // b, label)
    np.testing.assert_allclose(g["D"][:f], o["D"][:f], rtol=D_RTOL, atol=0, err_msg=label)
    assert np.max(np.abs(g["energy"][:f] - o["energy"][:f]), initial=0.0) <= E_ATOL, label
    return f


def check_replay(A, mu, tau, h, T, block, g, sample, label="", upto=0):
    """Refit sampled components (or blocks) from the GPU's own residual history.  A refit that
    differs must sit at a near-tie and the GPU's component (block) must be an equally good
    alternative.  Returns (replay result, number of differing samples)."""
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
            mism += 1
            gap = float(np.min(r["gap_o"][slots]))
            assert gap <= GAP_TOL, (
                f"{label}: component(s) {[i for i, ok in zip(rows, same) if not ok][:8]} differ "
                f"from the oracle refit; smallest gap in the block {gap:.3e}")
            check_alternative(A, mu, tau, h, T, block, g, int(s), label, r=r)
            continue
        np.testing.assert_allclose(g["D"][rows], r["Do"][slots], rtol=D_RTOL, atol=0,
                                   err_msg=f"{label}: D[{rows[0]}..]")
    er = r["energy_replay"]
    ok = ~np.isnan(er)
    assert np.max(np.abs(g["energy"][ok] - er[ok]), initial=0.0) <= E_ATOL, label
    return r, mism


def monotone(e):
    return bool(np.all(np.diff(e) >= -1e-12))


# ---- full-size reference runs of the oracle (tests/golden/make_full_fixtures.py) ----------

def factor_hashes(B, C):
    """64-bit BLAKE2b of (packed B row, packed C row) for each component."""
    B = np.ascontiguousarray(B).view(np.uint32)
    C = np.ascontiguousarray(C).view(np.uint32)
    out = np.empty(B.shape[0], dtype=np.uint64)
    for i in range(B.shape[0]):
        hsh = hashlib.blake2b(digest_size=8)
        hsh.update(B[i].tobytes())
        hsh.update(C[i].tobytes())
        out[i] = np.frombuffer(hsh.digest(), dtype=np.uint64)[0]
    return out


def input_sha(A, h):
    s = hashlib.sha256(np.ascontiguousarray(A, np.float32).tobytes())
    if h is not None:
        s.update(np.ascontiguousarray(h, np.float32).tobytes())
    return s.hexdigest()


def load_fixture(name, A, h):
    """The oracle's stored full-size run of workload ``name``; fails if the seeded generator no
    longer reproduces the input it was made from."""
    path = os.path.join(GOLDEN, f"full_{name}.npz")
    fx = dict(np.load(path, allow_pickle=False))
    assert str(fx["input_sha"]) == input_sha(A, h), (
        f"{name}: the input generator no longer reproduces the matrix the reference run was "
        "made from; rerun tests/golden/make_full_fixtures.py")
    return fx


def compare_with_fixture(g, fx):
    """Identical-prefix length, identical-component count, D and energy agreement of a GPU run
    against the oracle's stored full-size run."""
    hg = factor_hashes(g["B"], g["C"])
    same = hg == fx["hash"]
    k = len(same)
    bad = np.nonzero(~same)[0]
    f = int(bad[0]) if len(bad) else k
    dD = np.abs(g["D"].astype(np.float64) - fx["D"].astype(np.float64))
    relD = dD[same] / np.maximum(np.abs(fx["D"][same].astype(np.float64)), 1e-300)
    return dict(k=k, prefix=f, identical=int(same.sum()),
                D_exact=int(np.sum(g["D"][same] == fx["D"][same])),
                D_maxrel=float(relD.max(initial=0.0)),
                E_maxabs=float(np.max(np.abs(g["energy"] - fx["energy"]))))
