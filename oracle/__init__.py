"""fp64 CPU oracle for packed block-diagonal attention (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The product library never loads it; the two share no code.

The arithmetic lives in ``pfa_oracle.c`` (plain C, fp64, two passes per row: exact
row maximum first, then normaliser and weighted sum).  This module only builds and
marshals:

* ``varlen_fwd(q, k, v, cu_seqlens, scale, rows=None)`` -> ``(out, lse)``:
  ``out`` is ``[T, H, dv]`` fp64 and ``lse`` is ``[H, T]`` fp64 (natural log), or
  ``[n, H, dv]`` / ``[H, n]`` for a row sample ``rows``.
* ``varlen_fwd_qk(q, k, v, cu_q, cu_k, scale, rows=None)``: the same with separate query
  and key tables (queries of segment s attend the keys of segment s); a segment with
  queries but no keys gives a zero output and ``lse = -inf``.
* ``merge(o_a, lse_a, o_b, lse_b)`` -> ``(o, lse)``: attention over the union of two
  disjoint key sets from the results over each (fp64, see its docstring).
* ``varlen_bwd(q, k, v, dout, cu_seqlens, scale)`` -> ``(dq, dk, dv)`` fp64 ``[T, H, d]``:
  the gradients of the self-attention forward for upstream gradient ``dout``.
* ``rope(x, cos, sin)``: rotary position embedding of ``x`` [T, H, d] with per-token
  angle tables ``cos``, ``sin`` [T, d/2] (rotate-half pairs), fp64.
* ``qkv_rope_fwd(qkv, cu_seqlens, scale, cos=None, sin=None, rows=None)``: attention on a
  fused ``[T, 3, H, d]`` bf16 projection output, with q and k rotated and rounded to bf16
  first when tables are given.
* ``varlen_fwd_blocksparse(q, k, v, cu_seqlens, scale, layout, block_q, block_k, rows)``:
  restricted attention over listed key blocks per (segment, head, query block), numpy
  fp64; ``block_lists_from_mask`` turns a token mask into such lists.
* FP8 P.V variant: ``e4m3_round``, ``e4m3_encode``, ``e4m3_decode``, ``v_scale_exponent``,
  ``quantize_v_fp8`` (per (segment, head, channel) power-of-two scales, e4m3 codes),
  ``varlen_fwd_fp8pv_blocked`` (the blocked steps with FP8 weights and V, fp64) and
  ``fp8pv_error_bound`` (per-element bound against exact attention on the dequantised V).
* ``widen_bf16(bits)`` / ``round_bf16_bits(x)``: bf16 bits to fp64 and back (one
  rounding, ties to even).
* ``probs(q, k, cu_seqlens, scale, i, h)`` -> one row of the block-diagonal
  probability matrix over all ``T`` tokens (zero off-segment).

Inputs may be fp64 arrays or bf16 bit patterns (``uint16``), laid out ``[T, H, d]``
as in the packed_attention listing of the Mage-Flow page (section on native-resolution
sequence packing).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pfa_oracle.c")
# PFA_ORACLE_LIB selects another build of the same source (the sanitizer leg of the CPU
# tests loads an address/undefined-behaviour sanitized copy this way)
_SO = os.environ.get("PFA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

ELEM_F64 = 0
ELEM_BF16 = 1


def build(force: bool = True, sanitize: bool = False, path: str | None = None) -> str:
    """Compile ``liboracle.so`` with gcc (fp64, OpenMP, no FMA contraction).

    sanitize: build with AddressSanitizer and UndefinedBehaviorSanitizer (any report
    aborts), for the CPU tests' sanitizer leg; the process must preload gcc's libasan.
    path: where to write the library (default: next to this file)."""
    out = path or _SO
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
               "-std=c11", "-Wall", "-Wextra"]
        if sanitize:
            cmd += ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all"]
        cmd += ["-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.pfa_oracle_fwd.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, f64, vp, i64, vp, vp]
        lib.pfa_oracle_fwd.restype = i32
        lib.pfa_oracle_fwd_qk.argtypes = [i32, vp, vp, vp, vp, vp, i32, i32, i32, i32, f64, vp, i64,
                                          vp, vp]
        lib.pfa_oracle_fwd_qk.restype = i32
        lib.pfa_oracle_bwd.argtypes = [i32, vp, vp, vp, vp, vp, i32, i32, i32, f64, vp, vp, vp]
        lib.pfa_oracle_bwd.restype = i32
        lib.pfa_oracle_probs.argtypes = [i32, vp, vp, vp, i32, i32, i32, f64, i64, i32, vp]
        lib.pfa_oracle_probs.restype = i32
        lib.pfa_oracle_num_threads.argtypes = []
        lib.pfa_oracle_num_threads.restype = i32
        _lib = lib
    return _lib


def _kind(a: np.ndarray) -> int:
    if a.dtype == np.float64:
        return ELEM_F64
    if a.dtype == np.uint16:
        return ELEM_BF16
    raise TypeError(f"oracle inputs must be float64 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def varlen_fwd(q, k, v, cu_seqlens, scale: float, rows=None):
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    kind = _kind(q)
    if _kind(k) != kind or _kind(v) != kind:
        raise TypeError("q, k and v must share one element type")
    if q.ndim != 3 or k.shape != q.shape or v.ndim != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("expected q, k [T, H, d] and v [T, H, dv]")
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    T, H, d = q.shape
    dv = v.shape[2]
    num_seqs = cu.shape[0] - 1
    if num_seqs < 1 or int(cu[-1]) != T:
        raise ValueError("cu_seqlens must have >= 2 entries and end at T")
    if rows is None:
        n = T
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows_arr.shape[0]
    out = np.empty((n, H, dv), dtype=np.float64)
    lse = np.empty((H, n), dtype=np.float64)
    rc = _load().pfa_oracle_fwd(kind, _ptr(q), _ptr(k), _ptr(v), _ptr(cu), num_seqs, H, d, dv,
                                float(scale), _ptr(rows_arr) if rows_arr is not None else None,
                                n, _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return out, lse


def varlen_fwd_qk(q, k, v, cu_q, cu_k, scale: float, rows=None):
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    kind = _kind(q)
    if _kind(k) != kind or _kind(v) != kind:
        raise TypeError("q, k and v must share one element type")
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3 or k.shape[1:] != q.shape[1:] \
            or v.shape[:2] != k.shape[:2]:
        raise ValueError("expected q [Tq, H, d], k [Tk, H, d] and v [Tk, H, dv]")
    cq = np.ascontiguousarray(cu_q, dtype=np.int32)
    ck = np.ascontiguousarray(cu_k, dtype=np.int32)
    Tq, H, d = q.shape
    Tk = k.shape[0]
    dv = v.shape[2]
    num_seqs = cq.shape[0] - 1
    if num_seqs < 1 or ck.shape[0] != cq.shape[0] or int(cq[-1]) != Tq or int(ck[-1]) != Tk:
        raise ValueError("cu_q / cu_k must have the same length >= 2 and end at Tq / Tk")
    if rows is None:
        n = Tq
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows_arr.shape[0]
    out = np.empty((n, H, dv), dtype=np.float64)
    lse = np.empty((H, n), dtype=np.float64)
    rc = _load().pfa_oracle_fwd_qk(kind, _ptr(q), _ptr(k), _ptr(v), _ptr(cq), _ptr(ck), num_seqs,
                                   H, d, dv, float(scale),
                                   _ptr(rows_arr) if rows_arr is not None else None, n,
                                   _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return out, lse


def varlen_bwd(q, k, v, dout, cu_seqlens, scale: float):
    q, k, v, dout = (np.ascontiguousarray(a) for a in (q, k, v, dout))
    kind = _kind(q)
    if any(_kind(a) != kind for a in (k, v, dout)):
        raise TypeError("q, k, v and dout must share one element type")
    if q.ndim != 3 or any(a.shape != q.shape for a in (k, v, dout)):
        raise ValueError("expected q, k, v, dout all [T, H, d]")
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    T, H, d = q.shape
    if cu.shape[0] < 2 or int(cu[-1]) != T:
        raise ValueError("cu_seqlens must have >= 2 entries and end at T")
    dq, dk, dv = (np.empty((T, H, d), dtype=np.float64) for _ in range(3))
    rc = _load().pfa_oracle_bwd(kind, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(cu),
                                cu.shape[0] - 1, H, d, float(scale), _ptr(dq), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return dq, dk, dv


def rope(x, cos, sin):
    """Rotary position embedding, rotate-half pairing: for i < d/2,
        y[i]       = x[i] cos_i - x[i + d/2] sin_i
        y[i + d/2] = x[i + d/2] cos_i + x[i] sin_i,
    with the token's own angle table row (the same rotation for every head).  The pages
    place RoPE between the QKV projection and attention in the DiT block (Mage-Flow page,
    section on fusion opportunities in the DiT block) without fixing the variant; the
    rotate-half pairing and caller-supplied per-token tables (1-D, 2-D axial or any other
    position scheme reduces to them) are the reading taken.  fp64."""
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(cos, dtype=np.float64)[:, None, :]
    s = np.asarray(sin, dtype=np.float64)[:, None, :]
    half = x.shape[2] // 2
    a, b = x[:, :, :half], x[:, :, half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=2)


def qkv_rope_fwd(qkv_bits, cu_seqlens, scale: float, cos=None, sin=None, rows=None):
    """Attention on the fused projection output qkv [T, 3, H, d] (bf16 bits): q, k and v
    are its three consecutive chunks along the feature axis (the merged W_qkv projection
    of the Mage-Flow page, section on fusion opportunities in the DiT block, split into
    three with chunk(3, dim=-1)).  With angle tables, q and k are rotated (``rope``) and
    rounded to bf16, as a pipeline that stores them between the two steps would, before
    the attention of ``varlen_fwd``."""
    qkv = np.asarray(qkv_bits)
    if qkv.dtype != np.uint16 or qkv.ndim != 4 or qkv.shape[1] != 3:
        raise ValueError("expected qkv as bf16 bits [T, 3, H, d]")
    q, k, v = (np.ascontiguousarray(qkv[:, i]) for i in range(3))
    if (cos is None) != (sin is None):
        raise ValueError("give both angle tables or neither")
    if cos is not None:
        q = round_bf16_bits(rope(widen_bf16(q), cos, sin))
        k = round_bf16_bits(rope(widen_bf16(k), cos, sin))
    return varlen_fwd(q, k, v, cu_seqlens, scale, rows=rows)


def widen_bf16(bits):
    """bf16 bit patterns -> their exact fp64 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16_bits(x):
    """fp64 -> bf16 bit patterns, one rounding to nearest, ties to even, for values in
    bf16's normal range (and zero): bf16 keeps 8 significant bits, so x = m 2^e with
    0.5 <= |m| < 1 becomes rint(m 2^8) 2^(e-8); the result is exact in fp32, whose upper
    half is the bf16 pattern."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    r = np.ldexp(np.rint(m * 256.0), e - 8).astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def block_lists_from_mask(mask, block_q: int, block_k: int):
    """Block layout of a boolean token mask [n, n] (True = the pair is allowed): query block
    I lists key block J when any pair of the two blocks is allowed, the accounting of the
    SparseAttn article (section 04: a block with one allowed pair is computed whole).
    Returns (lists, stats): lists[I] = ascending key block indices; stats = allowed pairs,
    active blocks, computed positions (active blocks times block area) and utilisation."""
    m = np.asarray(mask, dtype=bool)
    n = m.shape[0]
    nq, nk = -(-n // block_q), -(-m.shape[1] // block_k)
    lists, active, computed = [], 0, 0
    for I in range(nq):
        rows = m[I * block_q:(I + 1) * block_q]
        row_list = []
        for J in range(nk):
            blk = rows[:, J * block_k:(J + 1) * block_k]
            if blk.any():
                row_list.append(J)
                active += 1
                computed += blk.size
        lists.append(row_list)
    pairs = int(m.sum())
    return lists, {"pairs": pairs, "active_blocks": active, "computed": computed,
                   "utilisation": pairs / computed if computed else 0.0}


def varlen_fwd_blocksparse(q, k, v, cu_seqlens, scale: float, layout, block_q: int = 256,
                           block_k: int = 64, rows=None):
    """Block-sparse restricted attention inside each segment.

    Query i of segment s (rows [a, a + L)) belongs to query block (i - a) // block_q; it
    attends exactly the keys j of its own segment whose key block (j - a) // block_k is
    listed for its (segment, head, query block), and the softmax is renormalised over
    that retained set (SparseAttn article, section 3.1: the restricted softmax; its
    section 05: a sliding-tile layout lets a query tile share a set of key tiles).
    ``layout[hl][s][qb]`` lists key block indices; ``len(layout)`` is 1 (one layout for
    every head) or H (head h uses ``layout[h]``).  Indices outside the segment's key
    blocks are ignored; a repeated index is an error.  A row with no retained key gets
    O = 0 and LSE = -inf.  Two passes per query block in fp64: exact row maximum, then
    normaliser and weighted sum; the products are numpy matmuls.  Returns (out, lse) as
    ``varlen_fwd`` does, for all rows or the sample ``rows``."""
    def as_f64(a):
        a = np.asarray(a)
        return widen_bf16(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float64)
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, _ = q.shape
    dv = v.shape[2]
    if len(layout) not in (1, H):
        raise ValueError("layout must hold one entry or one per head")
    want = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    slot = np.full(T, -1, dtype=np.int64)
    slot[want] = np.arange(want.shape[0])
    out = np.zeros((want.shape[0], H, dv))
    lse = np.full((H, want.shape[0]), -np.inf)
    for s in range(cu.shape[0] - 1):
        a, L = int(cu[s]), int(cu[s + 1] - cu[s])
        nkb = -(-L // block_k)
        for qb in range(-(-L // block_q)):
            r0, r1 = a + qb * block_q, a + min((qb + 1) * block_q, L)
            qrows = np.arange(r0, r1)[slot[r0:r1] >= 0]       # the requested rows only
            if qrows.size == 0:
                continue
            dst = slot[qrows]
            for h in range(H):
                listed = list(layout[h if len(layout) == H else 0][s][qb])
                if len(set(listed)) != len(listed):
                    raise ValueError(f"repeated key block in segment {s}, head {h}, query block {qb}")
                keys = [np.arange(a + J * block_k, a + min((J + 1) * block_k, L))
                        for J in listed if 0 <= J < nkb]
                if not keys:
                    continue                           # O = 0, LSE = -inf
                kk = np.concatenate(keys)
                sc = scale * (q[qrows, h] @ k[kk, h].T)
                m = sc.max(axis=1, keepdims=True)
                w = np.exp(sc - m)
                z = w.sum(axis=1, keepdims=True)
                out[dst, h] = (w @ v[kk, h]) / z
                lse[h, dst] = (m + np.log(z))[:, 0]
    return out, lse


# ------------------------------------------------------------------ FP8 P.V variant
# The FPS Attention slides (tool.lu deck on accelerating multimodal generation, slides
# 35-38) combine sliding-tile sparsity with FP8 attention: V quantised per channel, the
# probabilities P per tensor, and a dequantising FlashAttention.  Readings taken here (the
# slides give no formulas): FP8 is OCP e4m3 (3 mantissa bits, bias 7, largest finite 448,
# subnormal step 2^-9); V's scale is a power of two per (segment, head, channel), the
# smallest with max|V| / scale <= 448; P is scaled by the fixed per-tensor factor 2^8 (its
# range is (0, 1] under the online softmax) before rounding to e4m3.

E4M3_MAX = 448.0
P_SCALE_LOG2 = 8


def e4m3_round(x):
    """Round fp64 values (|x| <= 448) to the nearest e4m3 value, ties to even: 3 fraction
    bits for |x| >= 2^-6, a fixed step of 2^-9 below.  Returns the rounded fp64 values."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_round: |x| > 448")
    m, e = np.frexp(x)                       # x = m 2^e, 0.5 <= |m| < 1
    normal = np.abs(x) >= 2.0 ** -6
    r_norm = np.ldexp(np.rint(m * 16.0), e - 4)         # 4 significant bits
    r_sub = np.rint(x * 2.0 ** 9) * 2.0 ** -9
    return np.where(normal, r_norm, r_sub)


def e4m3_encode(x):
    """e4m3 codes (uint8) of values that are already e4m3 numbers (see e4m3_round)."""
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.abs(x)
    m, e = np.frexp(np.where(a > 0, a, 1.0))            # a = m 2^e
    normal = a >= 2.0 ** -6
    exp_field = np.where(normal, e - 1 + 7, 0)            # a = 1.f * 2^(e-1)
    frac = np.where(normal, np.rint((m * 2.0 - 1.0) * 8.0), np.rint(a * 2.0 ** 9))
    code = np.where(normal, (exp_field.astype(np.int64) << 3) | frac.astype(np.int64),
                    frac.astype(np.int64))
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_decode(codes):
    """Values of e4m3 codes (0x7F / 0xFF, the NaN codes, are not expected)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef, f = (c >> 3) & 0xF, c & 0x7
    val = np.where(ef == 0, f * 2.0 ** -9, np.ldexp(1.0 + f / 8.0, ef - 7))
    return sign * val


def v_scale_exponent(amax):
    """Smallest integer e with amax * 2^-e <= 448 (0 when amax is 0), raised to -126 when
    smaller so that the scale 2^e stays a normal fp32 number."""
    amax = np.asarray(amax, dtype=np.float64)
    m, E = np.frexp(np.where(amax > 0, amax, 1.0))      # amax = m 2^E, 0.5 <= m < 1
    e = np.maximum(np.where(m <= 0.875, E - 9, E - 8), -126)   # 448 = 0.875 * 2^9
    return np.where(amax > 0, e, 0).astype(np.int64)


def quantize_v_fp8(v_bits, cu_seqlens):
    """Per (segment, head, channel) power-of-two scaling of V and e4m3 rounding.
    Returns (codes uint8 [T, H, d], scales fp64 [S, H, d], each an exact power of two);
    V[t, h, c] is approximated by decode(codes[t, h, c]) * scales[s(t), h, c]."""
    v = widen_bf16(v_bits) if np.asarray(v_bits).dtype == np.uint16 else np.asarray(v_bits, np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, d = v.shape
    S = cu.shape[0] - 1
    codes = np.zeros((T, H, d), dtype=np.uint8)
    scales = np.ones((S, H, d))
    for s in range(S):
        a, b = int(cu[s]), int(cu[s + 1])
        if b <= a:
            continue
        e = v_scale_exponent(np.abs(v[a:b]).max(axis=0))      # [H, d]
        scales[s] = np.ldexp(1.0, e)
        codes[a:b] = e4m3_encode(e4m3_round(v[a:b] / scales[s][None]))
    return codes, scales


def dequantize_v_fp8(codes, scales, cu_seqlens):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    seg = np.searchsorted(cu[1:], np.arange(codes.shape[0]), side="right")
    return e4m3_decode(codes) * scales[seg]


def _retained_blocks(layout, L, s, h, H, qb, block_q, block_k):
    """Key blocks of query block qb of segment s, head h, in visiting order: every block in
    order without a layout, else the listed ones inside the segment (list order)."""
    nkb = -(-L // block_k)
    if layout is None:
        return list(range(nkb))
    listed = list(layout[h if len(layout) == H else 0][s][qb])
    if len(set(listed)) != len(listed):
        raise ValueError(f"repeated key block in segment {s}, head {h}, query block {qb}")
    return [J for J in listed if 0 <= J < nkb]


def varlen_fwd_fp8pv_blocked(q, k, v_codes, v_scales, cu_seqlens, scale: float, block: int = 64,
                             quantize: bool = True, rows=None, layout=None, block_q: int = 256):
    """The blocked online softmax (GigaPath-Flash page, section 3.2) with the P.V product in
    FP8, in fp64: per query row and 64-key block in order, the running maximum m (base 2)
    is raised to the block's maximum, accumulator and row sum are rescaled, the weights
    w = 2^8 2^(s log2(e) - m) are summed unrounded into l and rounded to e4m3 for the
    product with the e4m3 values of V; finally O = acc * scale_V / l and
    LSE = ln 2 (m - 8 + log2 l).  quantize=False keeps w unrounded (then the result is
    plain attention on the dequantised V).  With a block-sparse ``layout`` (see
    varlen_fwd_blocksparse; query blocks of block_q rows) only the listed key blocks are
    visited, in list order: the FPS Attention combination of sliding tiles and FP8.  A row
    with no retained key gets O = 0 and LSE = -inf."""
    q = widen_bf16(q) if np.asarray(q).dtype == np.uint16 else np.asarray(q, np.float64)
    k = widen_bf16(k) if np.asarray(k).dtype == np.uint16 else np.asarray(k, np.float64)
    v8 = e4m3_decode(v_codes)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, d = q.shape
    want = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    seg_of = np.searchsorted(cu[1:], want, side="right")
    out = np.zeros((want.shape[0], H, d))
    lse = np.full((H, want.shape[0]), -np.inf)
    c = scale / math.log(2.0)
    qblk = (want - cu[seg_of]) // block_q if layout is not None else np.zeros_like(want)
    for s, qb in sorted(set(zip(seg_of.tolist(), qblk.tolist()))):
        a, L = int(cu[s]), int(cu[s + 1] - cu[s])
        sel = np.nonzero((seg_of == s) & (qblk == qb))[0]
        qi = want[sel]
        for h in range(H):
            m = np.full(sel.shape[0], -np.inf)
            l = np.zeros(sel.shape[0])
            acc = np.zeros((sel.shape[0], d))
            for J in _retained_blocks(layout, L, s, h, H, qb, block_q, block):
                kk = np.arange(a + J * block, a + min((J + 1) * block, L))
                sc = (q[qi, h] @ k[kk, h].T) * c
                m_new = np.maximum(m, sc.max(axis=1))
                alpha = np.where(np.isneginf(m), 0.0, np.exp2(m - m_new))
                w = np.exp2(sc - m_new[:, None] + P_SCALE_LOG2)
                l = l * alpha + w.sum(axis=1)
                wq = e4m3_round(w) if quantize else w
                acc = acc * alpha[:, None] + wq @ v8[kk, h]
                m = m_new
            has = l > 0
            out[sel[has], h] = acc[has] * v_scales[s, h][None, :] / l[has, None]
            lse[h, sel[has]] = math.log(2.0) * (m[has] - P_SCALE_LOG2 + np.log2(l[has]))
    return out, lse


def fp8pv_error_bound(q, k, v_codes, v_scales, cu_seqlens, scale: float, rows=None, layout=None,
                      block_q: int = 256, block_k: int = 64):
    """Per-element bound on |O_fp8 - O| for O the exact attention on the dequantised V
    (over the retained keys when a block-sparse ``layout`` is given):
    O_fp8 = sum_j w8_j V_j / sum_j w_j with the same unrounded normaliser, and each e4m3
    weight is within max(2^-4 w_j, 2^-10) of w_j (half a step: relative 2^-4 for normal
    values, 2^-10 absolute below 2^-6).  With w_j = 2^8 p_j 2^(m_stage - M) <= 2^8 p_j,
    the error is at most sum_j (2^-4 p_j + 2^-18) |V_j| / sum_j p_j.  fp64, [n, H, d]."""
    q = widen_bf16(q) if np.asarray(q).dtype == np.uint16 else np.asarray(q, np.float64)
    k = widen_bf16(k) if np.asarray(k).dtype == np.uint16 else np.asarray(k, np.float64)
    vd = np.abs(dequantize_v_fp8(v_codes, v_scales, cu_seqlens))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, d = q.shape
    want = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    seg_of = np.searchsorted(cu[1:], want, side="right")
    qblk = (want - cu[seg_of]) // block_q if layout is not None else np.zeros_like(want)
    bound = np.zeros((want.shape[0], H, d))
    for s, qb in sorted(set(zip(seg_of.tolist(), qblk.tolist()))):
        a, L = int(cu[s]), int(cu[s + 1] - cu[s])
        sel = np.nonzero((seg_of == s) & (qblk == qb))[0]
        for h in range(H):
            blocks = _retained_blocks(layout, L, s, h, H, qb, block_q, block_k)
            if not blocks:
                continue
            kk = np.concatenate([np.arange(a + J * block_k, a + min((J + 1) * block_k, L)) for J in blocks])
            sc = scale * (q[want[sel], h] @ k[kk, h].T)
            p = np.exp(sc - sc.max(axis=1, keepdims=True))
            bound[sel, h] = (2.0 ** -4 * (p @ vd[kk, h]) + 2.0 ** -18 * vd[kk, h].sum(axis=0)) \
                / p.sum(axis=1, keepdims=True)
    return bound


def merge(o_a, lse_a, o_b, lse_b):
    """Attention over the union of two disjoint key sets A and B, from the results over
    each: with Z_X = exp(LSE_X) the partition sum over X, the union's partition sum is
    Z_A + Z_B and its output the Z-weighted mean of O_A and O_B (the identity behind the
    blocked update of the GigaPath-Flash page, section 3.2, applied to two finished
    blocks).  o_* are [n, H, dv], lse_* are [H, n]; fp64 throughout.  An empty set has
    LSE = -inf and contributes nothing; two empty sets give o = 0, lse = -inf."""
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    la = np.asarray(lse_a, dtype=np.float64)
    lb = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(la, lb)
    both_empty = np.isneginf(m)
    ms = np.where(both_empty, 0.0, m)
    za = np.exp(la - ms)                    # exp(-inf) = 0 for an empty side
    zb = np.exp(lb - ms)
    z = za + zb
    lse = np.where(both_empty, -np.inf, ms + np.log(np.where(both_empty, 1.0, z)))
    wa = np.where(both_empty, 0.0, za / np.where(both_empty, 1.0, z))
    wb = np.where(both_empty, 0.0, zb / np.where(both_empty, 1.0, z))
    o = wa.T[:, :, None] * o_a + wb.T[:, :, None] * o_b
    return o, lse


def probs(q, k, cu_seqlens, scale: float, i: int, h: int):
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    kind = _kind(q)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    T, H, d = q.shape
    p = np.empty(T, dtype=np.float64)
    rc = _load().pfa_oracle_probs(kind, _ptr(q), _ptr(k), _ptr(cu), cu.shape[0] - 1, H, d,
                                  float(scale), int(i), int(h), _ptr(p))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return p


def num_threads() -> int:
    return int(_load().pfa_oracle_num_threads())
