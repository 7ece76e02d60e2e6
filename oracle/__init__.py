"""Plain CPU oracle for the ExTernD decomposition engine.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product library never
loads it and shares no source with it; see ``externd_oracle.cpp`` for the method's steps and
the passages of the pages they follow (ExTernD review, Method and Key idea; pith.science
referee report, "What carries the argument", Prop. 1/2 and Eq. 3).

Functions here only marshal numpy arrays to the C++ oracle (``liboracle.so``, built with g++
by :func:`build`), plus the 2-bit unpacking of the packed ternary format.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "externd_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle with g++ (-O2, OpenMP, no FP contraction) into liboracle.so."""
    cmd = ["g++", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c++17",
           "-Wall", "-Wextra", _SRC, "-o", _LIB_PATH + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


class _Opts(ctypes.Structure):
    _fields_ = [
        ("threads", ctypes.c_int),
        ("safeguard", ctypes.c_int),
        ("k_limit", ctypes.c_int64),
        ("gaps", ctypes.POINTER(ctypes.c_double)),
        ("counters", ctypes.POINTER(ctypes.c_int64)),
        ("energy_explicit", ctypes.POINTER(ctypes.c_double)),
        ("residual_fp64", ctypes.c_int),
        ("block_engine", ctypes.c_int),
        ("energy_target", ctypes.c_double),
        ("used", ctypes.POINTER(ctypes.c_int64)),
        ("sweeps", ctypes.c_int),
        ("reverts", ctypes.POINTER(ctypes.c_int64)),
        ("ablation", ctypes.c_int),
    ]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64, f32, vp = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        lib.externd_oracle_rank.restype = i64
        lib.externd_oracle_rank.argtypes = [i64, i64, f32]
        lib.externd_oracle_words.restype = i64
        lib.externd_oracle_words.argtypes = [i64]
        lib.externd_oracle_splitmix64.restype = ctypes.c_uint64
        lib.externd_oracle_splitmix64.argtypes = [ctypes.c_uint64]
        lib.externd_oracle_sketch_sign.restype = ctypes.c_double
        lib.externd_oracle_sketch_sign.argtypes = [i64, i64, i64]
        lib.externd_oracle_block_targets.restype = ctypes.c_int
        lib.externd_oracle_block_targets.argtypes = [vp, i64, i64, vp, vp, vp, i64, ctypes.c_int, vp, vp]
        lib.externd_oracle_project.restype = ctypes.c_int
        lib.externd_oracle_project.argtypes = [vp, i64, f32, vp, vp, vp, vp, vp]
        lib.externd_oracle_decompose.restype = ctypes.c_int
        lib.externd_oracle_decompose.argtypes = [vp, i64, i64, f32, f32, vp, ctypes.c_int,
                                                 ctypes.c_int, vp, vp, vp, vp, vp]
        lib.externd_oracle_replay.restype = ctypes.c_int
        lib.externd_oracle_replay.argtypes = [vp, i64, i64, f32, f32, vp, ctypes.c_int,
                                              ctypes.c_int, vp, vp, vp, vp, i64, vp, vp, vp,
                                              vp, vp, vp, vp]
        lib.externd_oracle_matvec.restype = ctypes.c_int
        lib.externd_oracle_apply.argtypes = [vp, vp, vp, i64, i64, i64, vp, i64, vp, ctypes.c_int]
        lib.externd_oracle_matvec.argtypes = [vp, i64, i64, vp, vp, ctypes.c_int, vp,
                                              ctypes.c_int]
        lib.externd_oracle_explicit_energy.restype = ctypes.c_int
        lib.externd_oracle_explicit_energy.argtypes = [vp, i64, i64, vp, vp, vp, vp, i64, vp, i64,
                                                       vp, ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def rank(m: int, n: int, mu: float) -> int:
    """k = floor(mu * min(m, n) + 1e-9), or -1 if invalid."""
    return int(_load().externd_oracle_rank(m, n, mu))


def splitmix64(key: int) -> int:
    """First output of splitmix64 started from state `key` (the sketch's generator)."""
    return int(_load().externd_oracle_splitmix64(key & 0xFFFFFFFFFFFFFFFF))


def sketch_sign(s: int, c: int, j: int) -> float:
    """Entry (j, c) of block s's sign sketch: 1 for c = 0, else +-1 from splitmix64."""
    return float(_load().externd_oracle_sketch_sign(s, c, j))


def block_targets(A, U, V, h=None, naive: bool = False):
    """The block engine's targets for ternary U (bs x m) and V (bs x n): (X, Ft) with
    X = (U^T U + eps I)^-1 U^T A and Ft = (V^T H V + eps I)^-1 (A H V)^T."""
    A = np.ascontiguousarray(A, dtype=np.float32)
    m, n = A.shape
    U = np.ascontiguousarray(U, dtype=np.int8)
    V = np.ascontiguousarray(V, dtype=np.int8)
    bs = U.shape[0]
    assert U.shape == (bs, m) and V.shape == (bs, n)
    hh = _f32(h)
    X = np.zeros((bs, n), dtype=np.float64)
    Ft = np.zeros((bs, m), dtype=np.float64)
    rc = _load().externd_oracle_block_targets(_ptr(A), m, n, _ptr(hh), _ptr(U), _ptr(V), bs, int(naive),
                                              _ptr(X), _ptr(Ft))
    if rc != 0:
        raise ValueError("oracle block_targets failed")
    return X, Ft


def words(length: int) -> int:
    return (length + 15) // 16


def unpack(packed: np.ndarray, length: int) -> np.ndarray:
    """Packed 2-bit ternary rows (..., words) -> int8 rows (..., length).

    Element t is in bits 2(t%16)..2(t%16)+1 of word t//16; 00 -> 0, 01 -> +1, 11 -> -1.
    """
    packed = np.asarray(packed, dtype=np.uint32)
    shifts = (2 * np.arange(16, dtype=np.uint32))
    codes = (packed[..., :, None] >> shifts) & np.uint32(3)
    codes = codes.reshape(*packed.shape[:-1], packed.shape[-1] * 16)[..., :length]
    out = np.zeros(codes.shape, dtype=np.int8)
    out[codes == 1] = 1
    out[codes == 3] = -1
    return out


def project(x, tau: float = 0.0, h=None):
    """T_tau(x; h) -> (v int8, P, H, S, j, gap)."""
    x = _f32(x)
    h = _f32(h)
    L = x.shape[0]
    v = np.zeros(L, dtype=np.int8)
    out = np.zeros(3, dtype=np.float64)
    j = np.zeros(1, dtype=np.int64)
    gap = np.zeros(1, dtype=np.float64)
    _load().externd_oracle_project(_ptr(x), L, tau, _ptr(h), _ptr(v), _ptr(out), _ptr(j), _ptr(gap))
    return v, float(out[0]), float(out[1]), float(out[2]), int(j[0]), float(gap[0])


def _make_opts(threads, safeguard, k_limit, gaps, counters, eexp, residual_fp64,
               block_engine=False, energy_target=0.0, used=None, sweeps=0, reverts=None,
               ablation=0):
    o = _Opts()
    o.threads = int(threads)
    o.safeguard = int(bool(safeguard))
    o.k_limit = int(k_limit)
    dp, ip = ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)
    o.gaps = gaps.ctypes.data_as(dp) if gaps is not None else dp()
    o.counters = counters.ctypes.data_as(ip) if counters is not None else ip()
    o.energy_explicit = eexp.ctypes.data_as(dp) if eexp is not None else dp()
    o.residual_fp64 = int(bool(residual_fp64))
    o.block_engine = int(bool(block_engine))
    o.energy_target = float(energy_target)
    o.used = used.ctypes.data_as(ip) if used is not None else ip()
    o.sweeps = int(sweeps)
    o.reverts = reverts.ctypes.data_as(ip) if reverts is not None else ip()
    o.ablation = int(ablation)
    return o


def decompose(A, mu: float, tau: float = 0.0, h=None, als_iters: int = 4, block: int = 1,
              threads: int = 0, safeguard: bool = False, k_limit: int = 0,
              residual_fp64: bool = False, block_engine: bool = False,
              energy_target: float = 0.0, sweeps: int = 0, ablation: int = 0):
    """Free-running oracle decomposition.  Returns a dict with packed B, C, D, energy, gaps,
    counters (fallbacks, safeguard activations, ALS passes, zero components), the explicit
    final energy, k and ``used`` (components fitted before an energy-target stop; all of
    them without a target)."""
    A = np.ascontiguousarray(A, dtype=np.float32)
    h = _f32(h)
    m, n = A.shape
    k = rank(m, n, mu)
    if k < 1:
        raise ValueError("invalid rank")
    B = np.zeros((k, words(m)), dtype=np.uint32)
    C = np.zeros((k, words(n)), dtype=np.uint32)
    D = np.zeros(k, dtype=np.float32)
    energy = np.zeros(k, dtype=np.float64)
    gaps = np.full(k, np.inf)
    counters = np.zeros(4, dtype=np.int64)
    eexp = np.zeros(1, dtype=np.float64)
    used = np.zeros(1, dtype=np.int64)
    reverts = np.zeros(1, dtype=np.int64)
    o = _make_opts(threads, safeguard, k_limit, gaps, counters, eexp, residual_fp64,
                   block_engine, energy_target, used, sweeps, reverts, ablation)
    rc = _load().externd_oracle_decompose(_ptr(A), m, n, mu, tau, _ptr(h), als_iters, block,
                                          _ptr(B), _ptr(C), _ptr(D), _ptr(energy),
                                          ctypes.addressof(o))
    if rc != 0:
        raise ValueError(f"oracle decompose failed ({rc})")
    kk = k if k_limit <= 0 else min(k, k_limit)
    if (block not in (0, 1) or block_engine) and k_limit > 0:
        b = resolve_block(block, m, n, k)
        kk = min(k, -(-kk // b) * b)
    return dict(B=B[:kk], C=C[:kk], D=D[:kk], energy=energy[:kk], gaps=gaps[:kk],
                counters=counters, energy_explicit=float(eexp[0]), k=k, used=int(used[0]),
                reverts=int(reverts[0]))


def resolve_block(block: int, m: int, n: int, k: int) -> int:
    if block == -1:
        b = max(1, min(256, min(m, n) // 8))
    else:
        b = 1 if block <= 1 else block
    return min(b, k)


def replay(A, mu: float, tau: float, h, als_iters: int, block: int, B, C, D, sample,
           threads: int = 0, upto: int = 0):
    """Replay given factors; fit the sampled components (sequential) or blocks afresh.

    ``upto`` > 0 stops the walk after that many components (energy_replay is NaN beyond).
    Returns dict(Bo, Co, Do, gap_o, dec_o, energy_replay): the oracle's refit of each sample, its
    selection gaps and its energy decreases (units of |A|^2_H), and the energy curve of the given
    factors on the replayed residual.  For the block path each sample slot holds b components
    (rows sample_index*b .. +b of the factor arrays)."""
    A = np.ascontiguousarray(A, dtype=np.float32)
    h = _f32(h)
    m, n = A.shape
    k = rank(m, n, mu)
    b = resolve_block(block, m, n, k)
    B = np.ascontiguousarray(B, dtype=np.uint32)
    C = np.ascontiguousarray(C, dtype=np.uint32)
    D = np.ascontiguousarray(D, dtype=np.float32)
    assert B.shape == (k, words(m)) and C.shape == (k, words(n)) and D.shape == (k,)
    sample = np.ascontiguousarray(np.sort(np.asarray(sample, dtype=np.int64)))
    ns = sample.shape[0]
    slots = ns * b
    Bo = np.zeros((max(slots, 1), words(m)), dtype=np.uint32)
    Co = np.zeros((max(slots, 1), words(n)), dtype=np.uint32)
    Do = np.zeros(max(slots, 1), dtype=np.float32)
    go = np.full(max(slots, 1), np.inf)
    dec = np.zeros(max(slots, 1), dtype=np.float64)
    er = np.full(k, np.nan)
    o = _make_opts(threads, False, upto, None, None, None, False)
    rc = _load().externd_oracle_replay(_ptr(A), m, n, mu, tau, _ptr(h), als_iters, block,
                                       _ptr(B), _ptr(C), _ptr(D), _ptr(sample), ns, _ptr(Bo),
                                       _ptr(Co), _ptr(Do), _ptr(go), _ptr(dec), _ptr(er),
                                       ctypes.addressof(o))
    if rc != 0:
        raise ValueError(f"oracle replay failed ({rc})")
    return dict(Bo=Bo[:slots], Co=Co[:slots], Do=Do[:slots], gap_o=go[:slots], dec_o=dec[:slots],
                energy_replay=er, b=b, sample=sample)


def matvec(R, t, h=None, transpose: bool = False, threads: int = 0):
    """R^T t (transpose) or R (h * t), fp64 accumulation."""
    R = np.ascontiguousarray(R, dtype=np.float32)
    t = np.ascontiguousarray(t, dtype=np.int8)
    h = _f32(h)
    m, n = R.shape
    out = np.zeros(n if transpose else m, dtype=np.float64)
    _load().externd_oracle_matvec(_ptr(R), m, n, _ptr(t), _ptr(h), int(transpose), _ptr(out),
                                  threads)
    return out


def explicit_energy(A, h, B, C, D, at, threads: int = 0):
    """1 - |A - sum_{c<=i} D_c b_c c_c^T|^2_h / |A|^2_h after each component i in ``at``,
    recomputed in fp64 from the packed factors (the definition of the energy preserved)."""
    A = np.ascontiguousarray(A, dtype=np.float32)
    h = _f32(h)
    m, n = A.shape
    B = np.ascontiguousarray(B, dtype=np.uint32)
    C = np.ascontiguousarray(C, dtype=np.uint32)
    D = np.ascontiguousarray(D, dtype=np.float32)
    k = D.shape[0]
    assert B.shape == (k, words(m)) and C.shape == (k, words(n))
    at = np.ascontiguousarray(np.asarray(at, dtype=np.int64))
    out = np.zeros(max(1, at.shape[0]), dtype=np.float64)
    rc = _load().externd_oracle_explicit_energy(_ptr(A), m, n, _ptr(h), _ptr(B), _ptr(C), _ptr(D), k,
                                                _ptr(at), at.shape[0], _ptr(out), threads)
    if rc != 0:
        raise ValueError("oracle explicit_energy: bad arguments")
    return out[:at.shape[0]]


def apply(B, C, D, m: int, n: int, X, threads: int = 0):
    """Y = (B diag(D) C X^T)^T from packed factors (k x words(m), k x words(n)); X is n or batch x n."""
    B = np.ascontiguousarray(B, dtype=np.uint32)
    C = np.ascontiguousarray(C, dtype=np.uint32)
    D = np.ascontiguousarray(D, dtype=np.float32)
    X = np.ascontiguousarray(X, dtype=np.float32)
    single = X.ndim == 1
    X2 = X.reshape(1, -1) if single else X
    k = D.shape[0]
    assert X2.shape[1] == n and B.shape == (k, words(m)) and C.shape == (k, words(n))
    Y = np.zeros((X2.shape[0], m), dtype=np.float32)
    rc = _load().externd_oracle_apply(_ptr(B), _ptr(C), _ptr(D), k, m, n, _ptr(X2), X2.shape[0], _ptr(Y),
                                      threads)
    if rc != 0:
        raise ValueError(f"oracle apply failed ({rc})")
    return Y[0] if single else Y
