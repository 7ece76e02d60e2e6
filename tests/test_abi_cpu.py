"""The C-ABI library builds, loads and exports every symbol the public header declares; the
host-side validation paths answer without a GPU."""

import ctypes
import os
import re

import pytest

import expanded_rank_matrix_amd as erm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "externd.h")).read()
    return sorted(set(re.findall(r"\b(externd_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported():
    lib = erm.load()
    names = declared_symbols()
    assert "externd_decompose" in names and "externd_project" in names
    for name in names:
        assert hasattr(lib, name), name


def test_rank_and_words_host_only():
    assert erm.rank(2560, 2560, 3.0) == 7680
    assert erm.rank(9728, 2560, 2.0) == 5120
    assert erm.rank(2560, 9728, 3.0) == 7680
    assert erm.rank(64, 48, 2.0) == 96
    assert erm.rank(1024, 1024, 1.5) == 1536
    assert erm.rank(5, 5, 0.1) == -1
    assert erm.rank(0, 5, 1.0) == -1
    assert erm.rank(5, 5, float("nan")) == -1
    assert erm.packed_words(1) == 1 and erm.packed_words(16) == 1 and erm.packed_words(17) == 2


def test_status_strings():
    assert erm.status_string(0) == "EXTERND_OK"
    assert erm.status_string(-4) == "EXTERND_ENONFINITE"


def test_invalid_arguments_rejected_before_device_work():
    lib = erm.load()
    # null A: rejected on the host
    rc = lib.externd_decompose(None, 4, 4, 1.0, 0.0, None, 1, 1, None, None, None, None, None, None)
    assert rc == erm.EINVAL
    assert "null" in erm.last_error()
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    rc = lib.externd_decompose(fake, 4, 4, 1.0, 2.0, None, 1, 1, fake, fake, fake, fake, None, None)
    assert rc == erm.EINVAL and "tau" in erm.last_error()
    rc = lib.externd_decompose(fake, 4, 4, 1.0, 0.0, None, 0, 1, fake, fake, fake, fake, None, None)
    assert rc == erm.EINVAL and "als_iters" in erm.last_error()
    rc = lib.externd_decompose(fake, 20000, 4, 1.0, 0.0, None, 1, 1, fake, fake, fake, fake, None, None)
    assert rc == erm.EINVAL
    rc = lib.externd_decompose(fake, 4, 4, 0.01, 0.0, None, 1, 1, fake, fake, fake, fake, None, None)
    assert rc == erm.EINVAL and "mu" in erm.last_error()
    rc = lib.externd_project(None, 1, 4, 0.0, None, None, None, None)
    assert rc == erm.EINVAL


def test_apply_factors_arguments_rejected_before_device_work():
    lib = erm.load()
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    rc = lib.externd_apply_factors(None, fake, fake, 4, 4, 4, fake, 1, fake, None)
    assert rc == erm.EINVAL and "null" in erm.last_error()
    rc = lib.externd_apply_factors(fake, fake, fake, 0, 4, 4, fake, 1, fake, None)
    assert rc == erm.EINVAL
    rc = lib.externd_apply_factors(fake, fake, fake, 4, 4, 4, fake, 0, fake, None)
    assert rc == erm.EINVAL and "batch" in erm.last_error()
    rc = lib.externd_apply_factors(fake, fake, fake, 4, 4, 4, fake, 70000, fake, None)
    assert rc == erm.EINVAL and "batch" in erm.last_error()


def test_decompose_options_rejected_before_device_work():
    lib = erm.load()
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first

    def call(opt, block=1):
        return lib.externd_decompose_ex(fake, 8, 8, 2.0, 0.0, None, 1, block, fake, fake, fake,
                                        fake, ctypes.byref(opt), None, None)

    for t in (1.5, -0.1, float("nan"), float("inf")):
        assert call(erm.Options(t, 0, 0, 0)) == erm.EINVAL
        assert "energy_target" in erm.last_error()
    assert call(erm.Options(0.5, 2, 0, 0)) == erm.EINVAL and "safeguard" in erm.last_error()
    assert call(erm.Options(0.0, 0, -1, 0)) == erm.EINVAL and "sweeps" in erm.last_error()
    assert call(erm.Options(0.0, 0, 65, 0)) == erm.EINVAL and "sweeps" in erm.last_error()
    # the safeguard is defined for the sequential path; block 4 resolves to b = 4 here
    assert call(erm.Options(0.0, 1, 0, 0), block=4) == erm.EINVAL and "sequential" in erm.last_error()
    assert call(erm.Options(0.0, 0, 0, 4)) == erm.EINVAL and "ablation" in erm.last_error()
    assert call(erm.Options(0.0, 0, 0, 1)) == erm.EINVAL and "block path" in erm.last_error()
    assert call(erm.Options(0.0, 0, 0, 0, 2)) == erm.EINVAL and "residual_hbm" in erm.last_error()


def test_static_apply_arguments_rejected_before_device_work():
    lib = erm.load()
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    rc = lib.externd_apply_factors_static(None, fake, fake, 4, 4, 4, fake, 1, fake, None)
    assert rc == erm.EINVAL and "null" in erm.last_error()
    rc = lib.externd_apply_factors_static(fake, fake, fake, 4, 4, 4, fake, 0, fake, None)
    assert rc == erm.EINVAL and "batch" in erm.last_error()
    # 8 batch (k + m) bytes beyond the fixed 16 MiB workspace
    rc = lib.externd_apply_factors_static(fake, fake, fake, 7680, 2560, 2560, fake, 300, fake, None)
    assert rc == erm.EINVAL and "workspace" in erm.last_error()


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    A = torch.zeros((4, 4), dtype=torch.float32)
    with pytest.raises(ValueError):
        erm.decompose(A, 1.0)
    with pytest.raises(ValueError):
        erm.project(A)
