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
    assert set(declared_symbols()) == {"pfa_varlen_fwd", "pfa_varlen_fwd_qk", "pfa_varlen_fwd_qkv",
                                       "pfa_varlen_fwd_blocksparse", "pfa_check_block_layout",
                                       "pfa_quantize_v_fp8", "pfa_varlen_fwd_fp8pv",
                                       "pfa_varlen_fwd_blocksparse_fp8pv",
                                       "pfa_varlen_bwd", "pfa_varlen_bwd_noalloc", "pfa_attn_merge",
                                       "pfa_check_cu_seqlens", "pfa_status_string"}


def test_library_exports_every_declared_symbol(lib):
    from packed_varlen_flash_amd import _lib
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert set(declared_symbols()) == set(_lib.symbols())


def test_status_strings(lib):
    for code in range(-13, 1):
        assert lib.pfa_status_string(code)
    assert lib.pfa_status_string(-999) == b"unknown status"


def _fwd(lib, q=16, k=32, v=48, cu=64, num_seqs=1, max_seqlen=1, heads=1, head_dim=64, scale=1.0,
         out=80, lse=96):
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
    assert _fwd(lib, out=16) == -7
    assert _fwd(lib, lse=32) == -7
    assert _fwd(lib, lse=80) == -7
    # q, k, v and out move in 16-byte vectors; lse and the table one element at a time
    for name in ("q", "k", "v", "out"):
        for off in (2, 8):
            assert _fwd(lib, **{name: 256 + off}) == -12, (name, off)
    assert _fwd(lib, lse=258) == -12
    # a 4-byte aligned lse passes the alignment check (the size check after it fails)
    assert _fwd(lib, lse=100, num_seqs=2**30, heads=2**10, max_seqlen=2**20) == -11
    assert _fwd(lib, cu=66) == -12
    assert _fwd(lib, num_seqs=2**30, heads=2**10, max_seqlen=2**20) == -11
    assert _fwd(lib, heads=2**17 + 1, head_dim=64) == -11     # a row over 2^23 elements


def _fwd_qk(lib, q=16, k=32, v=48, cu_q=64, cu_k=128, num_seqs=1, max_q=1, max_k=1, heads=1,
            head_dim=64, scale=1.0, out=80, lse=96):
    return lib.pfa_varlen_fwd_qk(q, k, v, cu_q, cu_k, num_seqs, max_q, max_k, heads, head_dim, scale,
                                 out, lse, None)


def test_qk_argument_checks_run_before_any_hip_call(lib):
    assert _fwd_qk(lib, cu_k=None) == -1
    assert _fwd_qk(lib, cu_q=None) == -1
    assert _fwd_qk(lib, num_seqs=0) == -2
    assert _fwd_qk(lib, heads=0) == -3
    assert _fwd_qk(lib, max_q=0) == -4
    assert _fwd_qk(lib, max_k=0) == -4
    assert _fwd_qk(lib, head_dim=96) == -5
    assert _fwd_qk(lib, scale=float("nan")) == -6
    assert _fwd_qk(lib, out=128) == -7    # out aliases the key table
    assert _fwd_qk(lib, lse=128) == -7
    assert _fwd_qk(lib, lse=80) == -7
    for name in ("q", "k", "v", "out"):
        assert _fwd_qk(lib, **{name: 264}) == -12, name
    assert _fwd_qk(lib, cu_k=130) == -12
    assert _fwd_qk(lib, lse=97) == -12
    assert _fwd_qk(lib, num_seqs=2**30, heads=2**10, max_q=2**20) == -11


def _qkv(lib, qkv=16, cos=32, sin=48, cu=64, num_seqs=1, max_seqlen=1, heads=1, head_dim=64,
         scale=1.0, out=80, lse=96, k_rot=112):
    return lib.pfa_varlen_fwd_qkv(qkv, cos, sin, cu, num_seqs, max_seqlen, heads, head_dim, scale,
                                  out, lse, k_rot, None)


def test_qkv_argument_checks_run_before_any_hip_call(lib):
    assert _qkv(lib, qkv=None) == -1
    assert _qkv(lib, cu=None) == -1
    assert _qkv(lib, out=None) == -1
    assert _qkv(lib, cos=None) == -1            # one table without the other
    assert _qkv(lib, sin=None) == -1
    assert _qkv(lib, k_rot=None) == -1          # tables need the key workspace
    assert _qkv(lib, num_seqs=0) == -2
    assert _qkv(lib, heads=0) == -3
    assert _qkv(lib, max_seqlen=0) == -4
    assert _qkv(lib, head_dim=96) == -5
    assert _qkv(lib, scale=float("inf")) == -6
    assert _qkv(lib, out=16) == -7              # out is the fused input
    assert _qkv(lib, k_rot=32) == -7            # workspace is a table
    assert _qkv(lib, lse=80) == -7              # two outputs share a buffer
    assert _qkv(lib, k_rot=96) == -7
    assert _qkv(lib, qkv=18) == -12
    assert _qkv(lib, out=88) == -12
    assert _qkv(lib, k_rot=120) == -12
    assert _qkv(lib, sin=52) == -12
    assert _qkv(lib, heads=2**16, head_dim=64) == -11      # 3 * H * d over 2^23
    assert _qkv(lib, num_seqs=2**30, heads=2**10, max_seqlen=2**20) == -11


def _sparse(lib, q=16, k=32, v=48, cu=64, num_seqs=1, max_seqlen=1, heads=2, head_dim=64,
            scale=1.0, kv_ptr=80, kv_idx=96, nnz=1, layout_heads=1, out=112, lse=128):
    return lib.pfa_varlen_fwd_blocksparse(q, k, v, cu, num_seqs, max_seqlen, heads, head_dim, scale,
                                          kv_ptr, kv_idx, nnz, layout_heads, out, lse, None)


def test_blocksparse_argument_checks_run_before_any_hip_call(lib):
    for name in ("q", "k", "v", "cu", "out", "kv_ptr"):
        assert _sparse(lib, **{name: None}) == -1, name
    assert _sparse(lib, kv_idx=None) == -1                  # entries promised but no array
    assert _sparse(lib, num_seqs=0) == -2
    assert _sparse(lib, heads=0) == -3
    assert _sparse(lib, max_seqlen=0) == -4
    assert _sparse(lib, head_dim=80) == -5
    assert _sparse(lib, scale=-1.0) == -6
    assert _sparse(lib, nnz=-1) == -13
    assert _sparse(lib, layout_heads=3) == -13               # neither 1 nor heads
    assert _sparse(lib, layout_heads=0) == -13
    assert _sparse(lib, out=96) == -7                        # out is the index array
    assert _sparse(lib, lse=80) == -7
    assert _sparse(lib, lse=112) == -7
    for name in ("q", "k", "v", "out"):
        assert _sparse(lib, **{name: 264}) == -12, name
    for name in ("kv_ptr", "kv_idx", "lse", "cu"):
        assert _sparse(lib, **{name: 258}) == -12, name
    assert _sparse(lib, max_seqlen=65537) == -11             # beyond the LDS list
    assert _sparse(lib, heads=2**17, head_dim=128) == -11


def test_block_layout_validator():
    from packed_varlen_flash_amd import PfaError, block_layout_csr, pfa_check_block_layout
    lengths = [300, 0, 64, 1]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    good = [[[0, 1, 4], [2, 3]], [], [[0]], [[0]]]
    kv_ptr, kv_idx, lh = block_layout_csr([good], lengths, 300)
    assert lh == 1 and kv_ptr.shape[0] == 4 * 2 + 1 and kv_idx.tolist() == [0, 1, 4, 2, 3, 0, 0]
    pfa_check_block_layout(cu, 300, 2, 1, kv_ptr, kv_idx)
    per_head = [good, [[[4, 0], [1]], [], [[0]], [[0]]]]
    p2, i2, lh2 = block_layout_csr(per_head, lengths, 300)
    pfa_check_block_layout(cu, 300, 2, 2, p2, i2)
    with pytest.raises(PfaError) as e:
        pfa_check_block_layout(cu, 300, 3, 2, p2, i2)         # layout_heads neither 1 nor heads
    assert e.value.status == -13

    def bad(layout):
        p, i, l = block_layout_csr([layout], lengths, 300)
        with pytest.raises(PfaError) as e:
            pfa_check_block_layout(cu, 300, 2, l, p, i)
        assert e.value.status == -13

    bad([[[0, 1, 5], [2]], [], [[0]], [[0]]])      # block 5 is past the 300-token segment
    bad([[[0, 1, 1], [2]], [], [[0]], [[0]]])      # repeated block
    bad([[[0], []], [], [[0]], [[0]]])             # a query block with no keys
    bad([[[0], [1]], [], [[0], [0]], [[0]]])       # a query block the 64-token segment lacks
    bad([[[0], [-1]], [], [[0]], [[0]]])
    p, i, _ = block_layout_csr([good], lengths, 300)
    p_bad = p.copy()
    p_bad[-1] += 1                                 # does not end at nnz
    with pytest.raises(PfaError):
        pfa_check_block_layout(cu, 300, 2, 1, p_bad, i)
    p_bad = p.copy()
    p_bad[1], p_bad[2] = p_bad[2], p_bad[1]        # decreasing (0, 5, 3, ...)
    assert p_bad[1] > p_bad[2]
    with pytest.raises(PfaError):
        pfa_check_block_layout(cu, 300, 2, 1, p_bad, i)
    with pytest.raises(PfaError) as e:
        pfa_check_block_layout(cu, 200, 2, 1, np.zeros(5, np.int32), i)
    assert e.value.status == -8                    # cu_seqlens has a segment over max_seqlen


def _quant(lib, v=16, cu=32, num_seqs=1, heads=2, head_dim=64, v8=48, v_scale=64):
    return lib.pfa_quantize_v_fp8(v, cu, num_seqs, heads, head_dim, v8, v_scale, None)


def _fp8(lib, q=16, k=32, v8=48, v_scale=64, cu=80, num_seqs=1, max_seqlen=1, heads=2, head_dim=128,
         scale=1.0, out=96, lse=112):
    return lib.pfa_varlen_fwd_fp8pv(q, k, v8, v_scale, cu, num_seqs, max_seqlen, heads, head_dim, scale,
                                    out, lse, None)


def test_fp8_argument_checks_run_before_any_hip_call(lib):
    for name in ("v", "cu", "v8", "v_scale"):
        assert _quant(lib, **{name: None}) == -1, name
    assert _quant(lib, num_seqs=0) == -2
    assert _quant(lib, heads=0) == -3
    assert _quant(lib, head_dim=96) == -5
    assert _quant(lib, v8=16) == -7
    assert _quant(lib, v_scale=48) == -7
    assert _quant(lib, v=24) == -12                   # v not 16-byte aligned
    assert _quant(lib, v8=52) == -12
    assert _quant(lib, v_scale=66) == -12
    assert _quant(lib, num_seqs=2**20, heads=2**10) == -11
    for name in ("q", "k", "v8", "v_scale", "cu", "out"):
        assert _fp8(lib, **{name: None}) == -1, name
    assert _fp8(lib, num_seqs=0) == -2
    assert _fp8(lib, heads=0) == -3
    assert _fp8(lib, max_seqlen=0) == -4
    assert _fp8(lib, head_dim=32) == -5
    assert _fp8(lib, scale=0.0) == -6
    assert _fp8(lib, out=48) == -7
    assert _fp8(lib, lse=64) == -7
    assert _fp8(lib, v8=56) == -12
    for name in ("q", "k", "out"):
        assert _fp8(lib, **{name: 264}) == -12, name
    assert _fp8(lib, lse=258) == -12
    assert _quant(lib, cu=34) == -12
    assert _fp8(lib, heads=2**17, head_dim=128) == -11


def _fps(lib, q=16, k=32, v8=48, v_scale=64, cu=80, num_seqs=1, max_seqlen=1, heads=2, head_dim=128,
         scale=1.0, kv_ptr=96, kv_idx=112, nnz=1, layout_heads=1, out=128, lse=144):
    return lib.pfa_varlen_fwd_blocksparse_fp8pv(q, k, v8, v_scale, cu, num_seqs, max_seqlen, heads,
                                                head_dim, scale, kv_ptr, kv_idx, nnz, layout_heads,
                                                out, lse, None)


def test_fps_argument_checks_run_before_any_hip_call(lib):
    for name in ("q", "k", "v8", "v_scale", "cu", "out", "kv_ptr", "kv_idx"):
        assert _fps(lib, **{name: None}) == -1, name
    assert _fps(lib, kv_idx=None, nnz=0) != -1            # no entries, no index array needed
    assert _fps(lib, num_seqs=0) == -2
    assert _fps(lib, layout_heads=3) == -13
    assert _fps(lib, nnz=-2) == -13
    assert _fps(lib, out=112) == -7
    assert _fps(lib, lse=48) == -7
    assert _fps(lib, v_scale=68) == -12
    for name in ("q", "k", "out"):
        assert _fps(lib, **{name: 264}) == -12, name
    for name in ("kv_ptr", "kv_idx", "lse", "cu"):
        assert _fps(lib, **{name: 258}) == -12, name
    assert _fps(lib, max_seqlen=65537) == -11


def _merge(lib, o_a=16, lse_a=32, o_b=48, lse_b=64, total=1, heads=1, head_dim=64, out=16, lse=32):
    return lib.pfa_attn_merge(o_a, lse_a, o_b, lse_b, total, heads, head_dim, out, lse, None)


def test_merge_argument_checks_run_before_any_hip_call(lib):
    assert _merge(lib, o_a=None) == -1
    assert _merge(lib, lse_b=None) == -1
    assert _merge(lib, out=None) == -1
    assert _merge(lib, total=-1) == -11
    assert _merge(lib, heads=0) == -3
    assert _merge(lib, head_dim=32) == -5
    assert _merge(lib, out=32, lse=144) == -7    # out is an LSE input
    assert _merge(lib, out=144, lse=16) == -7    # lse is an O input
    assert _merge(lib, out=144, lse=144) == -7   # out and lse the same buffer
    for name in ("o_a", "o_b", "out"):
        assert _merge(lib, **{name: 264}) == -12, name
    for name in ("lse_a", "lse_b", "lse"):
        assert _merge(lib, **{name: 258}) == -12, name
    assert _merge(lib, total=0) == 0           # nothing to do, nothing launched
    assert _merge(lib, total=2**31, heads=1) == -11


def _bwd(lib, q=16, k=32, v=48, out=64, dout=80, lse=96, cu=112, num_seqs=1, max_seqlen=1, heads=1,
         head_dim=128, scale=1.0, dq=128, dk=144, dv=160, ws=176):
    return lib.pfa_varlen_bwd(q, k, v, out, dout, lse, cu, num_seqs, max_seqlen, heads, head_dim,
                              scale, dq, dk, dv, ws, None)


def test_bwd_argument_checks_run_before_any_hip_call(lib):
    for name in ("q", "k", "v", "out", "dout", "lse", "cu", "dq", "dk", "dv", "ws"):
        assert _bwd(lib, **{name: None}) == -1, name
    assert _bwd(lib, num_seqs=0) == -2
    assert _bwd(lib, heads=0) == -3
    assert _bwd(lib, max_seqlen=0) == -4
    assert _bwd(lib, head_dim=32) == -5
    assert _bwd(lib, scale=0.0) == -6
    assert _bwd(lib, dq=16) == -7         # output is an input
    assert _bwd(lib, ws=96) == -7         # workspace is the LSE
    assert _bwd(lib, dk=128) == -7        # two outputs share a buffer
    assert _bwd(lib, ws=160) == -7
    for name in ("q", "k", "v", "out", "dout", "dq", "dk", "dv"):
        assert _bwd(lib, **{name: 264}) == -12, name
    for name in ("lse", "cu", "ws"):
        assert _bwd(lib, **{name: 258}) == -12, name
    assert _bwd(lib, num_seqs=2**30, heads=2**10, max_seqlen=2**20) == -11


def _bwd_na(lib, q=16, k=32, v=48, out=64, dout=80, lse=96, cu=112, num_seqs=1, max_seqlen=1, T=1,
            heads=1, head_dim=128, scale=1.0, dq=128, dk=144, dv=160):
    return lib.pfa_varlen_bwd_noalloc(q, k, v, out, dout, lse, cu, num_seqs, max_seqlen, T, heads,
                                      head_dim, scale, dq, dk, dv, None)


def test_bwd_noalloc_argument_checks_run_before_any_hip_call(lib):
    for name in ("q", "k", "v", "out", "dout", "lse", "cu", "dq", "dk", "dv"):
        assert _bwd_na(lib, **{name: None}) == -1, name
    assert _bwd_na(lib, num_seqs=0) == -2
    assert _bwd_na(lib, heads=0) == -3
    assert _bwd_na(lib, head_dim=96) == -5
    assert _bwd_na(lib, dq=16) == -7
    assert _bwd_na(lib, dk=128) == -7
    assert _bwd_na(lib, dv=264) == -12
    # 2 * heads * T must fit the library's 2^23-value array
    assert _bwd_na(lib, T=-1) == -11
    assert _bwd_na(lib, heads=8, T=2**19 + 1) == -11
    assert _bwd_na(lib, heads=1, T=2**22 + 1) == -11


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


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


# ---- property tests of the host validators (hypothesis), against their definitions

from hypothesis import given, settings, strategies as st  # noqa: E402


@settings(max_examples=300, deadline=None)
@given(cu=st.lists(st.integers(-5, 300), min_size=2, max_size=20), mx=st.integers(1, 100))
def test_cu_seqlens_validator_matches_its_definition(lib, cu, mx):
    from packed_varlen_flash_amd import PfaError, pfa_check_cu_seqlens
    d = np.diff(cu)
    valid = cu[0] == 0 and bool(np.all(d >= 0)) and bool(np.all(d <= mx))
    if valid:
        assert pfa_check_cu_seqlens(cu, mx) == cu[-1]
    else:
        with pytest.raises(PfaError) as e:
            pfa_check_cu_seqlens(cu, mx)
        assert e.value.status == -8


@st.composite
def _sparse_layouts(draw):
    heads = draw(st.integers(1, 3))
    lh = draw(st.sampled_from(sorted({1, heads})))
    lengths = draw(st.lists(st.integers(0, 700), min_size=1, max_size=4))
    layout = []
    for _ in range(lh):
        segs = []
        for L in lengths:
            nkb = -(-L // 64)
            rows = []
            for _ in range(-(-L // 256)):
                rows.append(draw(st.lists(st.integers(0, nkb - 1), min_size=1, max_size=nkb, unique=True)))
            segs.append(rows)
        layout.append(segs)
    return heads, lengths, layout


@settings(max_examples=150, deadline=None)
@given(case=_sparse_layouts(), mutation=st.integers(0, 3), pick=st.integers(0, 10 ** 6))
def test_block_layout_validator_matches_its_definition(lib, case, mutation, pick):
    """Well-formed layouts (every existing query block lists distinct, in-range key blocks)
    are accepted; a duplicated entry, an out-of-range entry or an emptied query block is
    rejected."""
    from packed_varlen_flash_amd import PfaError, block_layout_csr, pfa_check_block_layout
    heads, lengths, layout = case
    mx = max(max(lengths), 1)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    rows = [(hl, s, qb) for hl in range(len(layout)) for s in range(len(lengths))
            for qb in range(len(layout[hl][s]))]
    if mutation and rows:
        hl, s, qb = rows[pick % len(rows)]
        row = layout[hl][s][qb]
        if mutation == 1:
            row.append(row[0])                     # listed twice
        elif mutation == 2:
            row.append(-(-lengths[s] // 64))       # one block past the segment's last
        else:
            row.clear()                            # a query block with no keys
    kv_ptr, kv_idx, lh = block_layout_csr(layout, lengths, mx)
    if mutation and rows:
        with pytest.raises(PfaError) as e:
            pfa_check_block_layout(cu, mx, heads, lh, kv_ptr, kv_idx)
        assert e.value.status == -13
    else:
        pfa_check_block_layout(cu, mx, heads, lh, kv_ptr, kv_idx)
