"""packed_varlen_flash_amd -- packed varlen attention forward on MI355X (gfx950).

A thin Python face over the C ABI of ``libpfa.so`` (declared in ``include/pfa.h``).
Every step of the computation runs in the library's HIP kernel; this module only checks
tensor metadata, allocates outputs with PyTorch when the caller does not pass them, and
hands raw pointers plus the current HIP stream to the library.  PyTorch is used for
device memory and streams, nothing else.
"""
from __future__ import annotations

import ctypes
import itertools

import numpy as np

from . import _lib

__all__ = ["pfa_varlen_fwd", "pfa_varlen_fwd_qk", "pfa_varlen_fwd_qkv", "pfa_varlen_bwd",
           "pfa_varlen_bwd_noalloc", "BWD_SCRATCH_FLOATS",
           "pfa_varlen_fwd_blocksparse", "block_layout_csr", "pfa_check_block_layout",
           "SPARSE_BLOCK_Q", "SPARSE_BLOCK_K", "pfa_quantize_v_fp8", "pfa_varlen_fwd_fp8pv",
           "pfa_varlen_fwd_blocksparse_fp8pv",
           "pfa_attn_merge",
           "pfa_check_cu_seqlens",
           "pfa_status_string", "PfaError", "LIB_PATH"]

LIB_PATH = _lib.LIB_PATH
SPARSE_BLOCK_Q = 256    # PFA_SPARSE_BLOCK_Q: query rows per block of a block-sparse layout
SPARSE_BLOCK_K = 64     # PFA_SPARSE_BLOCK_K: keys per key block
BWD_SCRATCH_FLOATS = 1 << 23   # PFA_BWD_SCRATCH_FLOATS: capacity of the backward's own array


class PfaError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"pfa status {status}: {pfa_status_string(status)}")


def pfa_status_string(status: int) -> str:
    return _lib.load().pfa_status_string(int(status)).decode()


def pfa_check_cu_seqlens(cu_host, max_seqlen: int) -> int:
    """Validate a host copy of cu_seqlens; return T or raise PfaError."""
    cu = np.ascontiguousarray(np.asarray(cu_host, dtype=np.int32))
    total = ctypes.c_int64(0)
    rc = _lib.load().pfa_check_cu_seqlens(cu.ctypes.data_as(ctypes.c_void_p), cu.shape[0] - 1,
                                          int(max_seqlen), ctypes.byref(total))
    if rc != 0:
        raise PfaError(rc)
    return int(total.value)


def _check_bf16(name, t, torch):
    if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous() or t.dim() != 3:
        raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor [T, H, d]")


def _check_table(name, cu, torch):
    if not cu.is_cuda or cu.dtype != torch.int32 or not cu.is_contiguous() or cu.dim() != 1:
        raise ValueError(f"{name} must be a contiguous 1-D int32 CUDA tensor")


def _check_buffer(name, t, device, dtype, shape):
    """A tensor the caller passes for the library to read or write: it must live on
    ``device`` (the first input's), have exactly ``dtype`` and ``shape`` and be contiguous,
    since the library receives only its address."""
    if t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_PLACEHOLDER_SLOTS = 64
_placeholders = {}
_next_slot = itertools.count()


def _ptr(t):
    """Device address of t for the C ABI.  A tensor with no elements has no storage, and
    the library rejects NULL; such a tensor gets a distinct 256-byte slot of a small
    per-device buffer instead.  The library reads and writes no rows there: a pack whose
    table holds no tokens (or no keys) gives the kernels no work on those buffers."""
    if t is None:
        return None
    if t.numel() > 0:
        return ctypes.c_void_p(t.data_ptr())
    import torch
    buf = _placeholders.get(t.device)
    if buf is None:
        buf = _placeholders[t.device] = torch.zeros(_PLACEHOLDER_SLOTS * 256, dtype=torch.uint8,
                                                    device=t.device)
    return ctypes.c_void_p(buf.data_ptr() + 256 * (next(_next_slot) % _PLACEHOLDER_SLOTS))


def pfa_varlen_fwd(q, k, v, cu_seqlens, max_seqlen: int, scale: float | None = None,
                   out=None, lse=None, want_lse: bool = True, stream=None):
    """Packed block-diagonal attention forward.

    q, k, v: bf16 CUDA tensors [T, H, d] (d = 64 or 128), contiguous.
    cu_seqlens: int32 CUDA tensor [num_seqs + 1].  max_seqlen: bound on segment lengths.
    Returns (out [T, H, d] bf16, lse [H, T] fp32 or None), enqueued on ``stream``
    (default: PyTorch's current stream).  T must equal cu_seqlens[-1]: the library takes T
    from the table on the device (it lays LSE out with that row stride), and this binding
    does not read the table on the host; pfa_check_cu_seqlens checks a host copy.
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor [T, H, d]")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    if not cu_seqlens.is_cuda or cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 CUDA tensor")
    for name, t in (("k", k), ("v", v), ("cu_seqlens", cu_seqlens)):
        if t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}")
    T, H, d = q.shape
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buffer("out", out, q.device, torch.bfloat16, q.shape)
    if lse is None and want_lse:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_buffer("lse", lse, q.device, torch.float32, (H, T))
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    rc = _lib.load().pfa_varlen_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), cu_seqlens.numel() - 1, int(max_seqlen), H, d,
        float(scale), _ptr(out), _ptr(lse),
        ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise PfaError(rc)
    return out, lse


def pfa_varlen_fwd_qk(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                      scale: float | None = None, out=None, lse=None, want_lse: bool = True,
                      stream=None):
    """Forward with separate query and key segment tables (queries of segment s attend
    the keys of segment s).  q: [Tq, H, d]; k, v: [Tk, H, d]; cu tables int32 [n + 1].
    Returns (out [Tq, H, d] bf16, lse [H, Tq] fp32 or None)."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(name, t, torch)
    if k.shape != v.shape or k.shape[1:] != q.shape[1:]:
        raise ValueError("k and v must be [Tk, H, d] with q's H and d")
    _check_table("cu_seqlens_q", cu_seqlens_q, torch)
    _check_table("cu_seqlens_k", cu_seqlens_k, torch)
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    for name, t in (("k", k), ("v", v), ("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}")
    Tq, H, d = q.shape
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buffer("out", out, q.device, torch.bfloat16, q.shape)
    if lse is None and want_lse:
        lse = torch.empty((H, Tq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_buffer("lse", lse, q.device, torch.float32, (H, Tq))
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    rc = _lib.load().pfa_varlen_fwd_qk(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
        cu_seqlens_q.numel() - 1, int(max_seqlen_q), int(max_seqlen_k), H, d, float(scale),
        _ptr(out), _ptr(lse), ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise PfaError(rc)
    return out, lse


def pfa_varlen_fwd_qkv(qkv, cu_seqlens, max_seqlen: int, scale: float | None = None,
                       rope_cos=None, rope_sin=None, out=None, lse=None, want_lse: bool = True,
                       k_rot=None, stream=None):
    """Self-attention forward read straight from a fused projection output.

    qkv: contiguous bf16 CUDA tensor [T, 3, H, d] (a [T, 3 * H * d] projection output
    viewed as such).  rope_cos, rope_sin: contiguous fp32 CUDA
    tensors [T, d / 2], or both None for no rotation; with them, q and k are rotated
    (rotate-half pairs) before attention and the rotated keys land in ``k_rot``
    ([T, H, d] bf16, allocated when not given).  Returns (out [T, H, d] bf16, lse [H, T]
    fp32 or None, k_rot or None)."""
    import torch

    if (not qkv.is_cuda or qkv.dtype != torch.bfloat16 or not qkv.is_contiguous() or qkv.dim() != 4
            or qkv.shape[1] != 3):
        raise ValueError("qkv must be a contiguous bf16 CUDA tensor [T, 3, H, d]")
    _check_table("cu_seqlens", cu_seqlens, torch)
    if cu_seqlens.device != qkv.device:
        raise ValueError(f"cu_seqlens must be on {qkv.device}")
    T, _, H, d = qkv.shape
    if (rope_cos is None) != (rope_sin is None):
        raise ValueError("pass both rope_cos and rope_sin, or neither")
    if rope_cos is not None:
        for name, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
            _check_buffer(name, t, qkv.device, torch.float32, (T, d // 2))
        if k_rot is None:
            k_rot = torch.empty((T, H, d), dtype=torch.bfloat16, device=qkv.device)
        else:
            _check_buffer("k_rot", k_rot, qkv.device, torch.bfloat16, (T, H, d))
    else:
        k_rot = None
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty((T, H, d), dtype=torch.bfloat16, device=qkv.device)
    else:
        _check_buffer("out", out, qkv.device, torch.bfloat16, (T, H, d))
    if lse is None and want_lse:
        lse = torch.empty((H, T), dtype=torch.float32, device=qkv.device)
    elif lse is not None:
        _check_buffer("lse", lse, qkv.device, torch.float32, (H, T))
    if stream is None:
        stream = torch.cuda.current_stream(qkv.device)
    rc = _lib.load().pfa_varlen_fwd_qkv(
        _ptr(qkv), _ptr(rope_cos), _ptr(rope_sin), _ptr(cu_seqlens), cu_seqlens.numel() - 1,
        int(max_seqlen), H, d, float(scale), _ptr(out), _ptr(lse), _ptr(k_rot),
        ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise PfaError(rc)
    return out, lse, k_rot


def block_layout_csr(layout, lengths, max_seqlen: int):
    """Pack nested lists layout[hl][s][qb] (key-block indices; len(layout) = 1 or heads)
    into the C ABI's CSR: row (s * layout_heads + hl) * qt_max + qb with qt_max =
    ceil(max_seqlen / SPARSE_BLOCK_Q).  Returns (kv_ptr, kv_idx, layout_heads) as int32
    numpy arrays plus the int; rows of query blocks a segment lacks stay empty."""
    lh = len(layout)
    qt_max = -(-int(max_seqlen) // SPARSE_BLOCK_Q)
    n = len(lengths)
    counts = np.zeros(n * lh * qt_max, dtype=np.int64)
    idx = []
    for s in range(n):
        for hl in range(lh):
            for qb, row in enumerate(layout[hl][s]):
                if qb >= qt_max:
                    raise ValueError("a segment has more query blocks than max_seqlen allows")
                counts[(s * lh + hl) * qt_max + qb] = len(row)
    for r in range(n * lh * qt_max):
        s, rem = divmod(r, lh * qt_max)
        hl, qb = divmod(rem, qt_max)
        rows = layout[hl][s]
        if qb < len(rows):
            idx.extend(int(j) for j in rows[qb])
    kv_ptr = np.zeros(counts.shape[0] + 1, dtype=np.int64)
    kv_ptr[1:] = np.cumsum(counts)
    if kv_ptr[-1] > np.iinfo(np.int32).max:
        raise ValueError("too many listed blocks")
    return kv_ptr.astype(np.int32), np.asarray(idx, dtype=np.int32), lh


def pfa_check_block_layout(cu_host, max_seqlen: int, heads: int, layout_heads: int, kv_ptr,
                           kv_idx) -> None:
    """Validate host copies of a block-sparse layout; raise PfaError when malformed."""
    cu = np.ascontiguousarray(np.asarray(cu_host, dtype=np.int32))
    p = np.ascontiguousarray(np.asarray(kv_ptr, dtype=np.int32))
    i = np.ascontiguousarray(np.asarray(kv_idx, dtype=np.int32))
    rows = (cu.shape[0] - 1) * int(layout_heads) * (-(-int(max_seqlen) // SPARSE_BLOCK_Q))
    if p.shape[0] != rows + 1:
        raise ValueError(f"kv_ptr must have {rows + 1} entries")
    rc = _lib.load().pfa_check_block_layout(
        cu.ctypes.data_as(ctypes.c_void_p), cu.shape[0] - 1, int(max_seqlen), int(heads),
        int(layout_heads), p.ctypes.data_as(ctypes.c_void_p),
        i.ctypes.data_as(ctypes.c_void_p) if i.size else None, int(i.shape[0]))
    if rc != 0:
        raise PfaError(rc)


def pfa_varlen_fwd_blocksparse(q, k, v, cu_seqlens, max_seqlen: int, kv_ptr, kv_idx,
                               layout_heads: int = 1, scale: float | None = None, out=None,
                               lse=None, want_lse: bool = True, stream=None):
    """Packed self-attention restricted to listed key blocks (see include/pfa.h).

    q, k, v: contiguous bf16 CUDA tensors [T, H, d]; kv_ptr, kv_idx: int32 CUDA tensors of
    the CSR layout (``block_layout_csr``); layout_heads: 1 or H.  Returns (out, lse)."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(name, t, torch)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    _check_table("cu_seqlens", cu_seqlens, torch)
    _check_table("kv_ptr", kv_ptr, torch)
    if kv_idx.numel() > 0:
        _check_table("kv_idx", kv_idx, torch)
    for name, t in (("k", k), ("v", v), ("cu_seqlens", cu_seqlens), ("kv_ptr", kv_ptr), ("kv_idx", kv_idx)):
        if t.numel() > 0 and t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}")
    T, H, d = q.shape
    rows = (cu_seqlens.numel() - 1) * int(layout_heads) * (-(-int(max_seqlen) // SPARSE_BLOCK_Q))
    if kv_ptr.numel() != rows + 1:
        raise ValueError(f"kv_ptr must have {rows + 1} entries for this max_seqlen and layout_heads")
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buffer("out", out, q.device, torch.bfloat16, q.shape)
    if lse is None and want_lse:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_buffer("lse", lse, q.device, torch.float32, (H, T))
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    rc = _lib.load().pfa_varlen_fwd_blocksparse(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), cu_seqlens.numel() - 1, int(max_seqlen), H, d,
        float(scale), _ptr(kv_ptr), _ptr(kv_idx) if kv_idx.numel() > 0 else None, int(kv_idx.numel()),
        int(layout_heads), _ptr(out), _ptr(lse), ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise PfaError(rc)
    return out, lse


def pfa_quantize_v_fp8(v, cu_seqlens, v8=None, v_scale=None, stream=None):
    """e4m3 codes of V with per (segment, head, channel) power-of-two scales (see
    include/pfa.h).  v: contiguous bf16 CUDA tensor [T, H, d].  Returns (v8 uint8 [T, H, d],
    v_scale fp32 [num_seqs, H, d])."""
    import torch

    _check_bf16("v", v, torch)
    _check_table("cu_seqlens", cu_seqlens, torch)
    if cu_seqlens.device != v.device:
        raise ValueError(f"cu_seqlens must be on {v.device}")
    T, H, d = v.shape
    n = cu_seqlens.numel() - 1
    if v8 is None:
        v8 = torch.empty((T, H, d), dtype=torch.uint8, device=v.device)
    else:
        _check_buffer("v8", v8, v.device, torch.uint8, (T, H, d))
    if v_scale is None:
        v_scale = torch.empty((n, H, d), dtype=torch.float32, device=v.device)
    else:
        _check_buffer("v_scale", v_scale, v.device, torch.float32, (n, H, d))
    if stream is None:
        stream = torch.cuda.current_stream(v.device)
    rc = _lib.load().pfa_quantize_v_fp8(_ptr(v), _ptr(cu_seqlens), n, H, d, _ptr(v8), _ptr(v_scale),
                                        ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise PfaError(rc)
    return v8, v_scale


def pfa_varlen_fwd_fp8pv(q, k, v8, v_scale, cu_seqlens, max_seqlen: int, scale: float | None = None,
                         out=None, lse=None, want_lse: bool = True, stream=None):
    """Packed self-attention with the P.V product in FP8 (see include/pfa.h): q, k bf16
    [T, H, d]; v8, v_scale from pfa_quantize_v_fp8.  Returns (out bf16 [T, H, d], lse)."""
    import torch

    for name, t in (("q", q), ("k", k)):
        _check_bf16(name, t, torch)
    if k.shape != q.shape:
        raise ValueError("q and k must have the same shape")
    _check_table("cu_seqlens", cu_seqlens, torch)
    T, H, d = q.shape
    n = cu_seqlens.numel() - 1
    for name, t in (("k", k), ("cu_seqlens", cu_seqlens)):
        if t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}")
    _check_buffer("v8", v8, q.device, torch.uint8, (T, H, d))
    _check_buffer("v_scale", v_scale, q.device, torch.float32, (n, H, d))
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buffer("out", out, q.device, torch.bfloat16, q.shape)
    if lse is None and want_lse:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_buffer("lse", lse, q.device, torch.float32, (H, T))
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    rc = _lib.load().pfa_varlen_fwd_fp8pv(
        _ptr(q), _ptr(k), _ptr(v8), _ptr(v_scale), _ptr(cu_seqlens), n, int(max_seqlen), H, d,
        float(scale), _ptr(out), _ptr(lse), ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise PfaError(rc)
    return out, lse


def pfa_varlen_fwd_blocksparse_fp8pv(q, k, v8, v_scale, cu_seqlens, max_seqlen: int, kv_ptr, kv_idx,
                                     layout_heads: int = 1, scale: float | None = None, out=None,
                                     lse=None, want_lse: bool = True, stream=None):
    """FPS Attention: block-sparse lists (as pfa_varlen_fwd_blocksparse) with P.V in FP8 (as
    pfa_varlen_fwd_fp8pv).  Returns (out bf16 [T, H, d], lse fp32 [H, T] or None)."""
    import torch

    for name, t in (("q", q), ("k", k)):
        _check_bf16(name, t, torch)
    if k.shape != q.shape:
        raise ValueError("q and k must have the same shape")
    _check_table("cu_seqlens", cu_seqlens, torch)
    _check_table("kv_ptr", kv_ptr, torch)
    if kv_idx.numel() > 0:
        _check_table("kv_idx", kv_idx, torch)
    T, H, d = q.shape
    n = cu_seqlens.numel() - 1
    for name, t in (("k", k), ("cu_seqlens", cu_seqlens), ("kv_ptr", kv_ptr), ("kv_idx", kv_idx)):
        if t.numel() > 0 and t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}")
    _check_buffer("v8", v8, q.device, torch.uint8, (T, H, d))
    _check_buffer("v_scale", v_scale, q.device, torch.float32, (n, H, d))
    rows = n * int(layout_heads) * (-(-int(max_seqlen) // SPARSE_BLOCK_Q))
    if kv_ptr.numel() != rows + 1:
        raise ValueError(f"kv_ptr must have {rows + 1} entries for this max_seqlen and layout_heads")
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buffer("out", out, q.device, torch.bfloat16, q.shape)
    if lse is None and want_lse:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_buffer("lse", lse, q.device, torch.float32, (H, T))
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    rc = _lib.load().pfa_varlen_fwd_blocksparse_fp8pv(
        _ptr(q), _ptr(k), _ptr(v8), _ptr(v_scale), _ptr(cu_seqlens), n, int(max_seqlen), H, d,
        float(scale), _ptr(kv_ptr), _ptr(kv_idx) if kv_idx.numel() > 0 else None, int(kv_idx.numel()),
        int(layout_heads), _ptr(out), _ptr(lse), ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise PfaError(rc)
    return out, lse


def pfa_attn_merge(o_a, lse_a, o_b, lse_b, out=None, lse=None, want_lse: bool = True,
                   stream=None):
    """Combine two results for the same queries over disjoint key sets (see pfa.h).
    o_*: bf16 [T, H, d]; lse_*: fp32 [H, T].  out / lse may be o_a / lse_a (in place).
    Returns (out, lse or None)."""
    import torch

    for name, t in (("o_a", o_a), ("o_b", o_b)):
        _check_bf16(name, t, torch)
    if o_b.shape != o_a.shape:
        raise ValueError("o_a and o_b must have the same shape")
    T, H, d = o_a.shape
    if o_b.device != o_a.device:
        raise ValueError(f"o_b must be on {o_a.device}")
    for name, t in (("lse_a", lse_a), ("lse_b", lse_b)):
        _check_buffer(name, t, o_a.device, torch.float32, (H, T))
    if out is None:
        out = torch.empty_like(o_a)
    else:
        _check_buffer("out", out, o_a.device, torch.bfloat16, o_a.shape)
    if lse is None and want_lse:
        lse = torch.empty((H, T), dtype=torch.float32, device=o_a.device)
    elif lse is not None:
        _check_buffer("lse", lse, o_a.device, torch.float32, (H, T))
    if stream is None:
        stream = torch.cuda.current_stream(o_a.device)
    rc = _lib.load().pfa_attn_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), T, H, d,
                                    _ptr(out), _ptr(lse), ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise PfaError(rc)
    return out, lse


def pfa_varlen_bwd(q, k, v, out, dout, lse, cu_seqlens, max_seqlen: int,
                   scale: float | None = None, dq=None, dk=None, dv=None, workspace=None,
                   stream=None):
    """Gradients (dq, dk, dv) of pfa_varlen_fwd for upstream gradient ``dout``.
    q, k, v, out, dout: bf16 [T, H, d]; lse: the forward's fp32 [H, T]; cu_seqlens int32.
    ``workspace`` (fp32 [2, H, T]) is allocated when not given."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _check_bf16(name, t, torch)
        if t.shape != q.shape:
            raise ValueError(f"{name} must have q's shape")
    _check_table("cu_seqlens", cu_seqlens, torch)
    T, H, d = q.shape
    for name, t in (("k", k), ("v", v), ("out", out), ("dout", dout), ("cu_seqlens", cu_seqlens)):
        if t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}")
    if lse is None:
        raise ValueError("lse must be the forward's contiguous fp32 [H, T]")
    _check_buffer("lse", lse, q.device, torch.float32, (H, T))
    if scale is None:
        scale = d ** -0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_buffer(name, t, q.device, torch.bfloat16, q.shape)
    if workspace is None:
        workspace = torch.empty((2, H, T), dtype=torch.float32, device=q.device)
    else:
        _check_buffer("workspace", workspace, q.device, torch.float32, (2, H, T))
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    rc = _lib.load().pfa_varlen_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(cu_seqlens),
        cu_seqlens.numel() - 1, int(max_seqlen), H, d, float(scale), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(workspace), ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise PfaError(rc)
    return dq, dk, dv


def pfa_varlen_bwd_noalloc(q, k, v, out, dout, lse, cu_seqlens, max_seqlen: int, total_tokens: int,
                           scale: float | None = None, dq=None, dk=None, dv=None, stream=None):
    """pfa_varlen_bwd without a workspace: the row statistics live in the library's own
    device array (see include/pfa.h), so with dq, dk and dv passed in nothing is allocated.
    total_tokens must equal cu_seqlens[-1]; 2 * H * total_tokens must not exceed
    BWD_SCRATCH_FLOATS.  Calls that overlap in time on one device race."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _check_bf16(name, t, torch)
        if t.shape != q.shape:
            raise ValueError(f"{name} must have q's shape")
    _check_table("cu_seqlens", cu_seqlens, torch)
    T, H, d = q.shape
    for name, t in (("k", k), ("v", v), ("out", out), ("dout", dout), ("cu_seqlens", cu_seqlens)):
        if t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}")
    if lse is None:
        raise ValueError("lse must be the forward's contiguous fp32 [H, T]")
    _check_buffer("lse", lse, q.device, torch.float32, (H, T))
    if int(total_tokens) != T:
        raise ValueError("total_tokens must be the packed token count (q.shape[0])")
    if scale is None:
        scale = d ** -0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_buffer(name, t, q.device, torch.bfloat16, q.shape)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    rc = _lib.load().pfa_varlen_bwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(cu_seqlens),
        cu_seqlens.numel() - 1, int(max_seqlen), int(total_tokens), H, d, float(scale), _ptr(dq),
        _ptr(dk), _ptr(dv), ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise PfaError(rc)
    return dq, dk, dv
