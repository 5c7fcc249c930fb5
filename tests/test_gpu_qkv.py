"""GPU parity of the fused-projection forward (pfa_varlen_fwd_qkv) against the fp64 oracle,
through the C ABI: q, k, v read in place from one [T, 3, H, d] tensor, optionally with
rotate-half RoPE on q and k (per-token angle tables)."""
import numpy as np
import pytest

import oracle
import pfa_workloads as W
from tests._gpu import assert_parity, compare, from_dev_bf16, say, to_dev

pytestmark = pytest.mark.gpu


def _tables_dev(cos, sin):
    import torch
    return (torch.from_numpy(np.ascontiguousarray(cos, np.float32)).to("cuda"),
            torch.from_numpy(np.ascontiguousarray(sin, np.float32)).to("cuda"))


def _run(wl, qkv_bits, cos, sin, label, want_lse=True):
    import torch
    from packed_varlen_flash_amd import pfa_varlen_fwd_qkv
    say(f"[gpu] pfa_varlen_fwd_qkv {label}: segs={wl.num_seqs} T={wl.total_tokens} H={wl.heads} "
        f"d={wl.head_dim} rope={cos is not None}")
    qkv = to_dev(qkv_bits)
    cu = torch.from_numpy(wl.cu_seqlens).to("cuda")
    c, s = _tables_dev(cos, sin) if cos is not None else (None, None)
    out, lse, k_rot = pfa_varlen_fwd_qkv(qkv, cu, wl.max_seqlen, wl.scale, c, s, want_lse=want_lse)
    torch.cuda.synchronize()
    return (from_dev_bf16(out), lse.cpu().numpy() if lse is not None else None,
            from_dev_bf16(k_rot) if k_rot is not None else None)


def _random_pack(seed, d, max_len=700):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 8))
    lengths = W.random_lengths(rng, n, max_len)
    if sum(lengths) == 0:
        lengths[0] = 1
    return W.make(lengths, 3, d, seed=seed, name=f"qkv{seed}")


@pytest.mark.parametrize("seed", range(6))
def test_fused_input_without_rotation_full(seed):
    wl = _random_pack(100 + seed, 64 if seed % 2 else 128)
    ob, lse, kr = _run(wl, W.fuse_qkv(wl.q, wl.k, wl.v), None, None, f"seed={seed} L={wl.lengths}")
    assert kr is None
    o_ref, l_ref = oracle.qkv_rope_fwd(W.fuse_qkv(wl.q, wl.k, wl.v), wl.cu_seqlens, wl.scale)
    assert_parity(compare(ob, lse, o_ref, l_ref), f"qkv seed={seed}")


@pytest.mark.parametrize("seed", range(6))
def test_fused_input_with_2d_rope_full(seed):
    wl = _random_pack(200 + seed, 64 if seed % 2 else 128)
    cos, sin = W.rope_tables_2d(wl.lengths, wl.head_dim)
    qkv = W.fuse_qkv(wl.q, wl.k, wl.v)
    ob, lse, kr = _run(wl, qkv, cos, sin, f"rope seed={seed} L={wl.lengths}")
    o_ref, l_ref = oracle.qkv_rope_fwd(qkv, wl.cu_seqlens, wl.scale, cos, sin)
    assert_parity(compare(ob, lse, o_ref, l_ref), f"qkv rope seed={seed}")
    # the rotated keys left in the workspace: evaluated in fp32 (error below 2^-22 of the
    # pair's magnitude) and rounded once to bf16, so within one bf16 step of the exactly
    # rounded value plus that fp32 error, and equal almost everywhere
    k = oracle.widen_bf16(wl.k)
    k_ref = oracle.round_bf16_bits(oracle.rope(k, cos, sin))
    a, b = W.bf16_to_f64(kr), W.bf16_to_f64(k_ref)
    h = wl.head_dim // 2
    pair = np.abs(k[..., :h]) + np.abs(k[..., h:])
    step = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(b), 1e-30))).astype(np.int64) - 7)
    assert np.all(np.abs(a - b) <= step + 2.0 ** -22 * np.concatenate([pair, pair], -1))
    assert np.mean(kr != k_ref) < 1e-3


def test_quarter_turns_match_plain_forward_on_rotated_inputs_bitwise():
    # whole quarter turns are exact in any precision, so the fused path must reproduce the
    # plain forward run on q and k rotated beforehand (by the oracle), bit for bit
    import torch
    from packed_varlen_flash_amd import pfa_varlen_fwd
    wl = W.make([300, 1, 0, 517, 64], 3, 128, seed=31)
    turns = np.random.default_rng(32).integers(0, 4, size=(wl.total_tokens, 64))
    cos = np.cos(turns * np.pi / 2).round().astype(np.float32)
    sin = np.sin(turns * np.pi / 2).round().astype(np.float32)
    ob, lse, kr = _run(wl, W.fuse_qkv(wl.q, wl.k, wl.v), cos, sin, "quarter turns")
    qr = oracle.round_bf16_bits(oracle.rope(oracle.widen_bf16(wl.q), cos, sin))
    kq = oracle.round_bf16_bits(oracle.rope(oracle.widen_bf16(wl.k), cos, sin))
    np.testing.assert_array_equal(kr, kq)
    cu = torch.from_numpy(wl.cu_seqlens).to("cuda")
    out2, lse2 = pfa_varlen_fwd(to_dev(qr), to_dev(kq), to_dev(wl.v), cu, wl.max_seqlen, wl.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ob, from_dev_bf16(out2))
    np.testing.assert_array_equal(lse, lse2.cpu().numpy())


def test_fused_input_matches_separate_tensors_bitwise():
    import torch
    from packed_varlen_flash_amd import pfa_varlen_fwd
    wl = W.make([1024, 33, 4096, 1], 4, 128, seed=33)
    ob, lse, _ = _run(wl, W.fuse_qkv(wl.q, wl.k, wl.v), None, None, "strided vs contiguous")
    cu = torch.from_numpy(wl.cu_seqlens).to("cuda")
    out2, lse2 = pfa_varlen_fwd(to_dev(wl.q), to_dev(wl.k), to_dev(wl.v), cu, wl.max_seqlen, wl.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ob, from_dev_bf16(out2))
    np.testing.assert_array_equal(lse, lse2.cpu().numpy())


def test_fused_c3_with_2d_rope_sampled():
    wl = W.generate("C3")
    cos, sin = W.rope_tables_2d(wl.lengths, wl.head_dim)
    qkv = W.fuse_qkv(wl.q, wl.k, wl.v)
    ob, lse, _ = _run(wl, qkv, cos, sin, "C3 2-D rope")
    rows = W.sample_rows(wl.cu_seqlens, stride=61, edge=64, full_upto=0)
    o_ref, l_ref = oracle.qkv_rope_fwd(qkv, wl.cu_seqlens, wl.scale, cos, sin, rows=rows)
    assert_parity(compare(ob[rows], lse[:, rows], o_ref, l_ref), f"C3 rope sampled {len(rows)} rows")


def test_without_lse_and_binding_checks():
    import torch
    from packed_varlen_flash_amd import pfa_varlen_fwd_qkv
    wl = W.make([70, 5], 2, 64, seed=34)
    ob, lse, _ = _run(wl, W.fuse_qkv(wl.q, wl.k, wl.v), None, None, "no lse", want_lse=False)
    assert lse is None
    o_ref, l_ref = oracle.qkv_rope_fwd(W.fuse_qkv(wl.q, wl.k, wl.v), wl.cu_seqlens, wl.scale)
    assert_parity(compare(ob, None, o_ref, l_ref), "qkv no lse")
    qkv = to_dev(W.fuse_qkv(wl.q, wl.k, wl.v))
    cu = torch.from_numpy(wl.cu_seqlens).to("cuda")
    c = torch.ones((wl.total_tokens, 32), device="cuda")
    with pytest.raises(ValueError):
        pfa_varlen_fwd_qkv(qkv, cu, wl.max_seqlen, rope_cos=c)             # one table only
    with pytest.raises(ValueError):
        pfa_varlen_fwd_qkv(qkv, cu, wl.max_seqlen, rope_cos=c[:, :16], rope_sin=c[:, :16])
    with pytest.raises(ValueError):
        pfa_varlen_fwd_qkv(qkv[:, :2], cu, wl.max_seqlen)                   # not [T, 3, H, d]


def test_many_segments_bitonic_schedule_with_rope():
    rng = np.random.default_rng(35)
    lengths = [int(x) for x in rng.integers(0, 200, size=600)]
    wl = W.make(lengths, 2, 128, seed=35, name="600 segments")
    cos, sin = W.rope_tables_2d(wl.lengths, 128)
    qkv = W.fuse_qkv(wl.q, wl.k, wl.v)
    ob, lse, _ = _run(wl, qkv, cos, sin, "600 segments, rope")
    o_ref, l_ref = oracle.qkv_rope_fwd(qkv, wl.cu_seqlens, wl.scale, cos, sin)
    assert_parity(compare(ob, lse, o_ref, l_ref), "qkv 600 segments")


def test_poison_in_other_segments_does_not_leak():
    wl = W.make([300, 700, 90], 2, 128, seed=36)
    cos, sin = W.rope_tables_2d(wl.lengths, 128)
    qkv = W.fuse_qkv(wl.q, wl.k, wl.v)
    ob, lse, _ = _run(wl, qkv, cos, sin, "clean")
    a, b = int(wl.cu_seqlens[1]), int(wl.cu_seqlens[2])
    bad = qkv.copy()
    bad[:a] = 0x7FC0
    bad[b:] = 0x7F80
    ob2, lse2, _ = _run(wl, bad, cos, sin, "poisoned neighbours")
    np.testing.assert_array_equal(ob2[a:b], ob[a:b])
    np.testing.assert_array_equal(lse2[:, a:b], lse[:, a:b])
