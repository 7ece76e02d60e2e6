"""Write the oracle's full-size reference runs of the workloads to tests/golden/full_<name>.npz.

Calls only the CPU oracle (``oracle/``) on the seeded synthetic inputs of
``expanded_rank_matrix_amd.inputs``; nothing here comes from the GPU path.  For each workload it
stores:

* ``input_sha``: sha256 of A (and h) as generated, so a test notices a changed generator;
* ``hash``: one 64-bit BLAKE2b digest per component over (B row, C row), the packed ternary
  factors as the C ABI emits them, and ``D``, the scales;
* ``energy``: the oracle's energy curve (fp64 bookkeeping);
* ``gaps``: each component's smallest selection gap (diagnostics at a divergence);
* ``explicit_at`` / ``explicit``: the energy preserved recomputed from the oracle's own factors
  (``oracle.explicit_energy``) after components 256 q - 1 and after the last one;
* ``counters`` and ``energy_explicit_final`` (the oracle's explicit final energy of its fp32
  residual).

Usage: python tests/golden/make_full_fixtures.py [workload ...] [--threads N]
(all four large workloads by default; the block workloads take minutes of CPU time each).
"""

from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from expanded_rank_matrix_amd import inputs  # noqa: E402
from tests._parity import factor_hashes, input_sha  # noqa: E402

WORKLOADS = ("lowrank1024", "attn2560", "mlp9728x2560", "down2560x9728")


def checkpoints(k):
    """Components after which the energy is recomputed explicitly: 256 q - 1, and the last."""
    at = list(range(255, k, 256))
    if not at or at[-1] != k - 1:
        at.append(k - 1)
    return np.asarray(at, dtype=np.int64)


def fixture_path(name):
    return os.path.join(HERE, f"full_{name}.npz")


def make(name, threads=0):
    c = inputs.CONFIGS[name]
    A, h = inputs.make_input(name)
    t0 = time.time()
    o = oracle.decompose(A, c["mu"], c["tau"], h, c["als_iters"], c["block"], threads=threads)
    secs = time.time() - t0
    at = checkpoints(o["k"])
    expl = oracle.explicit_energy(A, h, o["B"], o["C"], o["D"], at, threads=threads)
    np.savez_compressed(fixture_path(name), input_sha=np.array(input_sha(A, h)),
                        hash=factor_hashes(o["B"], o["C"]), D=o["D"], energy=o["energy"],
                        gaps=o["gaps"].astype(np.float32), explicit_at=at, explicit=expl,
                        counters=o["counters"], energy_explicit_final=np.float64(o["energy_explicit"]))
    print(f"{name}: k={o['k']} final energy {o['energy'][-1]:.12f} ({secs:.1f} s)", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workloads", nargs="*", default=list(WORKLOADS))
    ap.add_argument("--threads", type=int, default=0)
    args = ap.parse_args()
    for name in args.workloads:
        make(name, args.threads)


if __name__ == "__main__":
    main()
