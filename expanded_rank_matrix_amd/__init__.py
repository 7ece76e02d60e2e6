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
        ("residual_lds", ctypes.c_int64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class Options(ctypes.Structure):
    _fields_ = [
        ("energy_target", ctypes.c_double),
        ("safeguard", ctypes.c_int),
        ("sweeps", ctypes.c_int),
        ("ablation", ctypes.c_int),
        ("residual_hbm", ctypes.c_int),
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


def _require(t, dtype, name, shape=None, device=None):
    """t as the C ABI will read or write it: a contiguous CUDA tensor of ``dtype`` (any of them
    when a tuple), on ``device`` and of exactly ``shape`` when given.  The library gets raw
    pointers and sizes, so a short or mistyped buffer would be read or written out of bounds."""
    if t is None:
        return None
    dtypes = dtype if isinstance(dtype, tuple) else (dtype,)
    if not (t.is_cuda and t.dtype in dtypes and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous CUDA tensor of {' or '.join(map(str, dtypes))}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def decompose(A, mu: float, tau: float = 0.0, h=None, als_iters: int = 4, block: int = 1,
              stream=None, out=None, energy_target: float = 0.0, safeguard: bool = False,
              sweeps: int = 0, ablation: int = 0, residual_hbm: bool = False):
    """Run externd_decompose (externd_decompose_ex when an option is set) on a device fp32
    matrix A (m x n).

    Returns dict(B, C, D, energy, stats): B (k x words(m)) and C (k x words(n)) packed uint32
    stored in int32 tensors, D fp32 (k), energy fp64 (k), stats dict.  ``out`` may supply
    preallocated outputs as a dict with the same keys.  ``energy_target`` in (0, 1] stops after
    the first component whose energy reaches it (stats["components_used"]); ``safeguard`` turns
    on the best single-entry safeguard (sequential path); ``sweeps`` refinement sweeps refit
    every component after the greedy pass; ``ablation`` switches parts of the method off for
    ablation studies (1: block targets without decorrelation, 2: unweighted V-step projection);
    ``residual_hbm`` keeps the sequential path's residual in HBM even where it fits in LDS."""
    import torch

    A = _require(A, torch.float32, "A")
    if A.dim() != 2:
        raise ValueError("A must be a 2-d matrix")
    m, n = A.shape
    dev = A.device
    h = _require(h, torch.float32, "h", shape=(n,), device=dev)
    k = rank(m, n, mu)
    if k < 1:
        raise ExterndError(EINVAL, "mu gives k < 1")
    if out is None:
        out = dict(
            B=torch.empty((k, packed_words(m)), dtype=torch.int32, device=dev),
            C=torch.empty((k, packed_words(n)), dtype=torch.int32, device=dev),
            D=torch.empty(k, dtype=torch.float32, device=dev),
            energy=torch.empty(k, dtype=torch.float64, device=dev),
        )
    words32 = (torch.int32, torch.uint32)
    _require(out["B"], words32, "out['B']", shape=(k, packed_words(m)), device=dev)
    _require(out["C"], words32, "out['C']", shape=(k, packed_words(n)), device=dev)
    _require(out["D"], torch.float32, "out['D']", shape=(k,), device=dev)
    _require(out["energy"], torch.float64, "out['energy']", shape=(k,), device=dev)
    st = Stats()
    if energy_target or safeguard or sweeps or ablation or residual_hbm:
        opt = Options(float(energy_target), int(bool(safeguard)), int(sweeps), int(ablation),
                      int(bool(residual_hbm)))
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
    if X.dim() != 2:
        raise ValueError("X must be count x L")
    count, L = X.shape
    h = _require(h, torch.float32, "h", shape=(L,), device=X.device)
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
    if R.dim() != 2:
        raise ValueError("R must be a 2-d matrix")
    m, n = R.shape
    t = _require(t, torch.int8, "t", shape=(m if transpose else n,), device=R.device)
    if h is not None and transpose:
        raise ValueError("h weights the U-step product R (h .* t) only")
    h = _require(h, torch.float32, "h", shape=(n,), device=R.device)
    out = torch.empty(n if transpose else m, dtype=torch.float64, device=R.device)
    rc = load().externd_matvec(_dev_ptr(R), m, n, _dev_ptr(t), _dev_ptr(h), int(transpose),
                               _dev_ptr(out), _stream_ptr(stream))
    _check(rc)
    return out


def _apply_args(B, C, D, m, n, X, out):
    """Validated (B, C, D, k, X2, Y, single) for the inference entry points."""
    import torch

    D = _require(D, torch.float32, "D")
    if D.dim() != 1:
        raise ValueError("D must be a vector of k scales")
    k = D.shape[0]
    dev = D.device
    words32 = (torch.int32, torch.uint32)
    _require(B, words32, "B", shape=(k, packed_words(m)), device=dev)
    _require(C, words32, "C", shape=(k, packed_words(n)), device=dev)
    X = _require(X, torch.float32, "X", device=dev)
    single = X.dim() == 1
    X2 = X.reshape(1, -1) if single else X
    if X2.dim() != 2 or X2.shape[1] != n:
        raise ValueError("X must be n or batch x n")
    Y = out if out is not None else torch.empty((X2.shape[0], m), dtype=torch.float32, device=dev)
    _require(Y, torch.float32, "out", device=dev)
    if Y.numel() != X2.shape[0] * m:
        raise ValueError("out must hold batch x m values")
    return B, C, D, k, X2, Y, single


def apply_factors(B, C, D, m: int, n: int, X, stream=None, out=None):
    """Y = (B diag(D) C X^T)^T from packed factors (as returned by decompose) for X (n or batch x n,
    fp32, device); returns Y (m or batch x m, fp32).  Enqueued on the stream without waiting (the
    library keeps a workspace per device and stream)."""
    B, C, D, k, X2, Y, single = _apply_args(B, C, D, m, n, X, out)
    rc = load().externd_apply_factors(_dev_ptr(B), _dev_ptr(C), _dev_ptr(D), k, m, n, _dev_ptr(X2),
                                      X2.shape[0], _dev_ptr(Y), _stream_ptr(stream))
    _check(rc)
    return Y[0] if single else Y.reshape(X2.shape[0], m)


def apply_factors_static(B, C, D, m: int, n: int, X, stream=None, out=None):
    """externd_apply_factors_static: as apply_factors, with the library's fixed per-GPU workspace
    (no device allocation) and without waiting for the stream; synchronise before reading Y."""
    B, C, D, k, X2, Y, single = _apply_args(B, C, D, m, n, X, out)
    rc = load().externd_apply_factors_static(_dev_ptr(B), _dev_ptr(C), _dev_ptr(D), k, m, n, _dev_ptr(X2),
                                             X2.shape[0], _dev_ptr(Y), _stream_ptr(stream))
    _check(rc)
    return Y[0] if single else Y.reshape(X2.shape[0], m)


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
