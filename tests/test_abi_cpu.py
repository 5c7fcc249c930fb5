"""Host-side checks of the C ABI: the library loads, exports what include/pfa.h declares,
and rejects bad arguments before touching the HIP runtime (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pfa.h")


@pytest.fixture(scope="module")
def lib():
    from packed_varlen_flash_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from packed_varlen_flash_amd import build
        build.build()
    return _lib.load()


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"PFA_API\s+[\w\s\*]+?\b(pfa_\w+)\s*\(", text)


def test_header_declares_the_abi():
    assert set(declared_symbols()) == {"pfa_varlen_fwd", "pfa_check_cu_seqlens", "pfa_status_string"}


def test_library_exports_every_declared_symbol(lib):
    from packed_varlen_flash_amd import _lib
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert set(declared_symbols()) == set(_lib.symbols())


def test_status_strings(lib):
    for code in range(-11, 1):
        assert lib.pfa_status_string(code)
    assert lib.pfa_status_string(-999) == b"unknown status"


def _fwd(lib, q=1, k=2, v=3, cu=4, num_seqs=1, max_seqlen=1, heads=1, head_dim=64, scale=1.0,
         out=5, lse=6):
    return lib.pfa_varlen_fwd(q, k, v, cu, num_seqs, max_seqlen, heads, head_dim, scale, out, lse, None)


def test_argument_checks_run_before_any_hip_call(lib):
    # Fake non-NULL pointers are never dereferenced: every case fails a check first.
    assert _fwd(lib, q=None) == -1
    assert _fwd(lib, out=None) == -1
    assert _fwd(lib, cu=None) == -1
    assert _fwd(lib, num_seqs=0) == -2
    assert _fwd(lib, heads=0) == -3
    assert _fwd(lib, max_seqlen=0) == -4
    for hd in (0, 32, 96, 256):
        assert _fwd(lib, head_dim=hd) == -5
    for sc in (0.0, -1.0, float("inf"), float("nan")):
        assert _fwd(lib, scale=sc) == -6
    assert _fwd(lib, out=1) == -7
    assert _fwd(lib, lse=2) == -7
    assert _fwd(lib, lse=5) == -7
    assert _fwd(lib, num_seqs=2**30, heads=2**10, max_seqlen=2**20) == -11


def test_host_validator(lib):
    from packed_varlen_flash_amd import PfaError, pfa_check_cu_seqlens
    assert pfa_check_cu_seqlens([0, 3, 3, 10], 7) == 10
    assert pfa_check_cu_seqlens([0, 1], 1) == 1
    for bad, mx in (([1, 3], 5), ([0, 3, 2], 5), ([0, 9], 8)):
        with pytest.raises(PfaError) as e:
            pfa_check_cu_seqlens(bad, mx)
        assert e.value.status == -8
    arr = np.array([0, 4], np.int32)
    assert lib.pfa_check_cu_seqlens(arr.ctypes.data_as(ctypes.c_void_p), 0, 4, None) == -2
    assert lib.pfa_check_cu_seqlens(arr.ctypes.data_as(ctypes.c_void_p), 1, 0, None) == -4
    assert lib.pfa_check_cu_seqlens(None, 1, 4, None) == -1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from packed_varlen_flash_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.load()
