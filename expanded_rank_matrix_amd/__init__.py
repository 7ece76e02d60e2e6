"""MI355X-native ExTernD decomposition engine: thin Python binding of libexternd.so.

Every step of the decomposition runs in the library's HIP kernels; this module only marshals
torch device tensors (device memory and the current stream) to the C ABI declared in
``include/externd.h``.  There is no CPU fallback: if the library is missing the calls raise.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libexternd.so")

OK, EINVAL, ENOMEM, EDEVICE, ENONFINITE = 0, -1, -2, -3, -4

_lib = None


class ExterndError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status) if _lib else status}: {message}")
        self.status = status


class Stats(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_int64),
        ("passes", ctypes.c_int64),
        ("early_exits", ctypes.c_int64),
        ("fallback_inits", ctypes.c_int64),
        ("zero_components", ctypes.c_int64),
        ("block", ctypes.c_int64),
        ("energy_final_explicit", ctypes.c_double),
        ("seconds", ctypes.c_double),
        ("kernel_ms", ctypes.c_double),
        ("bytes_algorithmic", ctypes.c_double),
        ("flops_algorithmic", ctypes.c_double),
        ("components_used", ctypes.c_int64),
        ("safeguard_activations", ctypes.c_int64),
        ("sweep_reverts", ctypes.c_int64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class Options(ctypes.Structure):
    _fields_ = [
        ("energy_target", ctypes.c_double),
        ("safeguard", ctypes.c_int),
        ("sweeps", ctypes.c_int),
        ("ablation", ctypes.c_int),
    ]


def load():
    """Load libexternd.so (built by ``expanded_rank_matrix_amd.build``); raise if missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                              "python -m expanded_rank_matrix_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        i64, f32, vp, ci = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int
        lib.externd_rank.restype = i64
        lib.externd_rank.argtypes = [i64, i64, f32]
        lib.externd_packed_words.restype = i64
        lib.externd_packed_words.argtypes = [i64]
        lib.externd_decompose.restype = ci
        lib.externd_decompose.argtypes = [vp, i64, i64, f32, f32, vp, ci, ci, vp, vp, vp, vp, vp,
                                          ctypes.POINTER(Stats)]
        lib.externd_decompose_ex.restype = ci
        lib.externd_decompose_ex.argtypes = [vp, i64, i64, f32, f32, vp, ci, ci, vp, vp, vp, vp,
                                             ctypes.POINTER(Options), vp, ctypes.POINTER(Stats)]
        lib.externd_project.restype = ci
        lib.externd_project.argtypes = [vp, i64, i64, f32, vp, vp, vp, vp]
        lib.externd_matvec.restype = ci
        lib.externd_matvec.argtypes = [vp, i64, i64, vp, vp, ci, vp, vp]
        lib.externd_apply_factors.restype = ci
        lib.externd_apply_factors.argtypes = [vp, vp, vp, i64, i64, i64, vp, i64, vp, vp]
        lib.externd_apply_factors_static.restype = ci
        lib.externd_apply_factors_static.argtypes = [vp, vp, vp, i64, i64, i64, vp, i64, vp, vp]
        lib.externd_status_string.restype = ctypes.c_char_p
        lib.externd_status_string.argtypes = [ci]
        lib.externd_last_error.restype = ctypes.c_char_p
        lib.externd_last_error.argtypes = []
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().externd_status_string(status).decode()


def last_error() -> str:
    return load().externd_last_error().decode()


def _check(status: int):
    if status != OK:
        raise ExterndError(status, last_error())


def rank(m: int, n: int, mu: float) -> int:
    return int(load().externd_rank(m, n, mu))


def packed_words(length: int) -> int:
    return int(load().externd_packed_words(length))


def _dev_ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _require(t, dtype, name):
    import torch

    if t is None:
        return None
    if not (t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")
    return t


def decompose(A, mu: float, tau: float = 0.0, h=None, als_iters: int = 4, block: int = 1,
              stream=None, out=None, energy_target: float = 0.0, safeguard: bool = False,
              sweeps: int = 0, ablation: int = 0):
    """Run externd_decompose (externd_decompose_ex when an option is set) on a device fp32
    matrix A (m x n).

    Returns dict(B, C, D, energy, stats): B (k x words(m)) and C (k x words(n)) packed uint32
    stored in int32 tensors, D fp32 (k), energy fp64 (k), stats dict.  ``out`` may supply
    preallocated outputs as a dict with the same keys.  ``energy_target`` in (0, 1] stops after
    the first component whose energy reaches it (stats["components_used"]); ``safeguard`` turns
    on the best single-entry safeguard (sequential path); ``sweeps`` refinement sweeps refit
    every component after the greedy pass; ``ablation`` switches parts of the method off for
    ablation studies (1: block targets without decorrelation, 2: unweighted V-step projection)."""
    import torch

    A = _require(A, torch.float32, "A")
    h = _require(h, torch.float32, "h")
    m, n = A.shape
    k = rank(m, n, mu)
    if k < 1:
        raise ExterndError(EINVAL, "mu gives k < 1")
    dev = A.device
    if out is None:
        out = dict(
            B=torch.empty((k, packed_words(m)), dtype=torch.int32, device=dev),
            C=torch.empty((k, packed_words(n)), dtype=torch.int32, device=dev),
            D=torch.empty(k, dtype=torch.float32, device=dev),
            energy=torch.empty(k, dtype=torch.float64, device=dev),
        )
    st = Stats()
    if energy_target or safeguard or sweeps or ablation:
        opt = Options(float(energy_target), int(bool(safeguard)), int(sweeps), int(ablation))
        rc = load().externd_decompose_ex(_dev_ptr(A), m, n, mu, tau, _dev_ptr(h), als_iters, block,
                                         _dev_ptr(out["B"]), _dev_ptr(out["C"]),
                                         _dev_ptr(out["D"]), _dev_ptr(out["energy"]),
                                         ctypes.byref(opt), _stream_ptr(stream), ctypes.byref(st))
    else:
        rc = load().externd_decompose(_dev_ptr(A), m, n, mu, tau, _dev_ptr(h), als_iters, block,
                                      _dev_ptr(out["B"]), _dev_ptr(out["C"]), _dev_ptr(out["D"]),
                                      _dev_ptr(out["energy"]), _stream_ptr(stream),
                                      ctypes.byref(st))
    _check(rc)
    res = dict(out)
    res["stats"] = st.as_dict()
    res["k"] = k
    return res


def project(X, tau: float = 0.0, h=None, stream=None):
    """Ternary projection of each row of X (count x L, fp32, device).
    Returns (V int8 count x L, PHC fp64 count x 3)."""
    import torch

    X = _require(X, torch.float32, "X")
    h = _require(h, torch.float32, "h")
    count, L = X.shape
    V = torch.empty((count, L), dtype=torch.int8, device=X.device)
    PHC = torch.empty((count, 3), dtype=torch.float64, device=X.device)
    rc = load().externd_project(_dev_ptr(X), count, L, tau, _dev_ptr(h), _dev_ptr(V), _dev_ptr(PHC),
                                _stream_ptr(stream))
    _check(rc)
    return V, PHC


def matvec(R, t, h=None, transpose: bool = False, stream=None):
    """R^T t (transpose) or R (h .* t) with fp64 accumulation; R fp32 (m x n), t int8."""
    import torch

    R = _require(R, torch.float32, "R")
    t = _require(t, torch.int8, "t")
    h = _require(h, torch.float32, "h")
    m, n = R.shape
    out = torch.empty(n if transpose else m, dtype=torch.float64, device=R.device)
    rc = load().externd_matvec(_dev_ptr(R), m, n, _dev_ptr(t), _dev_ptr(h), int(transpose),
                               _dev_ptr(out), _stream_ptr(stream))
    _check(rc)
    return out


def apply_factors(B, C, D, m: int, n: int, X, stream=None, out=None):
    """Y = (B diag(D) C X^T)^T from packed factors (as returned by decompose) for X (n or batch x n,
    fp32, device); returns Y (m or batch x m, fp32)."""
    import torch

    D = _require(D, torch.float32, "D")
    X = _require(X, torch.float32, "X")
    for t, name in ((B, "B"), (C, "C")):
        if not (t.is_cuda and t.dtype in (torch.int32, torch.uint32) and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous 32-bit CUDA tensor of packed words")
    k = D.shape[0]
    if B.shape != (k, packed_words(m)) or C.shape != (k, packed_words(n)):
        raise ValueError("B, C must be k x packed_words(m), k x packed_words(n)")
    single = X.dim() == 1
    X2 = X.reshape(1, -1) if single else X
    if X2.shape[1] != n:
        raise ValueError("X must have n columns")
    Y = out if out is not None else torch.empty((X2.shape[0], m), dtype=torch.float32, device=X.device)
    rc = load().externd_apply_factors(_dev_ptr(B), _dev_ptr(C), _dev_ptr(D), k, m, n, _dev_ptr(X2),
                                      X2.shape[0], _dev_ptr(Y), _stream_ptr(stream))
    _check(rc)
    return Y[0] if single else Y


def apply_factors_static(B, C, D, m: int, n: int, X, stream=None, out=None):
    """externd_apply_factors_static: as apply_factors, with the library's fixed per-GPU workspace
    (no device allocation) and without waiting for the stream; synchronise before reading Y."""
    import torch

    D = _require(D, torch.float32, "D")
    X = _require(X, torch.float32, "X")
    for t, name in ((B, "B"), (C, "C")):
        if not (t.is_cuda and t.dtype in (torch.int32, torch.uint32) and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous 32-bit CUDA tensor of packed words")
    k = D.shape[0]
    if B.shape != (k, packed_words(m)) or C.shape != (k, packed_words(n)):
        raise ValueError("B, C must be k x packed_words(m), k x packed_words(n)")
    single = X.dim() == 1
    X2 = X.reshape(1, -1) if single else X
    if X2.shape[1] != n:
        raise ValueError("X must have n columns")
    Y = out if out is not None else torch.empty((X2.shape[0], m), dtype=torch.float32, device=X.device)
    if Y.dtype != torch.float32 or not Y.is_contiguous() or Y.numel() != X2.shape[0] * m:
        raise ValueError("out must be a contiguous fp32 tensor of batch x m values")
    rc = load().externd_apply_factors_static(_dev_ptr(B), _dev_ptr(C), _dev_ptr(D), k, m, n, _dev_ptr(X2),
                                             X2.shape[0], _dev_ptr(Y), _stream_ptr(stream))
    _check(rc)
    return Y[0] if single else Y


def unpack(packed, length: int) -> np.ndarray:
    """Packed 2-bit ternary rows (..., words) -> int8 (..., length); accepts torch or numpy.

    Element t is in bits 2(t%16)..2(t%16)+1 of word t//16; 00 -> 0, 01 -> +1, 11 -> -1."""
    if hasattr(packed, "cpu"):
        packed = packed.cpu().numpy()
    w = np.asarray(packed).view(np.uint32)
    codes = (w[..., :, None] >> (2 * np.arange(16, dtype=np.uint32))) & np.uint32(3)
    codes = codes.reshape(*w.shape[:-1], w.shape[-1] * 16)[..., :length]
    out = np.zeros(codes.shape, dtype=np.int8)
    out[codes == 1] = 1
    out[codes == 3] = -1
    return out


def sparsity_and_bpw(B_packed, C_packed, m: int, n: int):
    """Zero fractions of B and C and the effective bits per weight of the mask+sign storage
    model, (m k (2 - s_B) + k n (2 - s_C)) / (m n), the pages' Eq. 5 accounting with D absorbed
    (pith.science free parameters, Eq. 5)."""
    U = unpack(B_packed, m)
    V = unpack(C_packed, n)
    k = U.shape[0]
    sB = 1.0 - np.count_nonzero(U) / (m * k)
    sC = 1.0 - np.count_nonzero(V) / (k * n)
    bpw = (m * k * (2.0 - sB) + k * n * (2.0 - sC)) / (m * n)
    return sB, sC, bpw
