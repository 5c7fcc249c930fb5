"""ctypes view of libpfa.so: the C ABI declared in include/pfa.h, nothing more."""
from __future__ import annotations

import ctypes
import os

# PFA_LIB selects another build of the same sources (the sanitizer leg of the CPU tests
# loads a copy whose host code carries address/undefined-behaviour sanitizers this way)
LIB_PATH = os.environ.get("PFA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpfa.so")

# Every symbol include/pfa.h declares, with its ctypes signature.
_SIGNATURES = {
    "pfa_varlen_fwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p]),
    "pfa_varlen_fwd_qk": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]),
    "pfa_varlen_fwd_qkv": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int] * 4 +
                           [ctypes.c_float] + [ctypes.c_void_p] * 4),
    "pfa_varlen_fwd_blocksparse": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int] * 4 +
                                   [ctypes.c_float] + [ctypes.c_void_p] * 2 +
                                   [ctypes.c_int] * 2 + [ctypes.c_void_p] * 3),
    "pfa_check_block_layout": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_int] * 4 +
                               [ctypes.c_void_p] * 2 + [ctypes.c_int]),
    "pfa_quantize_v_fp8": (ctypes.c_int, [ctypes.c_void_p] * 2 + [ctypes.c_int] * 3 +
                           [ctypes.c_void_p] * 3),
    "pfa_varlen_fwd_fp8pv": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 +
                             [ctypes.c_float] + [ctypes.c_void_p] * 3),
    "pfa_varlen_fwd_blocksparse_fp8pv": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 +
                                         [ctypes.c_float] + [ctypes.c_void_p] * 2 +
                                         [ctypes.c_int] * 2 + [ctypes.c_void_p] * 3),
    "pfa_attn_merge": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "pfa_varlen_bwd": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int] * 4 +
                       [ctypes.c_float] + [ctypes.c_void_p] * 5),
    "pfa_varlen_bwd_noalloc": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int] * 2 +
                               [ctypes.c_int64] + [ctypes.c_int] * 2 + [ctypes.c_float] +
                               [ctypes.c_void_p] * 4),
    "pfa_check_cu_seqlens": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_void_p]),
    "pfa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}

_lib = None


def load():
    """Load libpfa.so; raise if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it first (python -m packed_varlen_flash_amd.build "
                "or __graft_entry__.build()); there is no CPU fallback")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def symbols():
    return list(_SIGNATURES)
