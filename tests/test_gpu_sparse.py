"""GPU parity of the block-sparse forward (pfa_varlen_fwd_blocksparse) against the fp64
oracle, through the C ABI: each 256-query block of a segment attends only its listed
64-key blocks, with the softmax renormalised over them."""
import dataclasses

import numpy as np
import pytest

import oracle
import pfa_workloads as W
from tests._gpu import assert_parity, compare, from_dev_bf16, say, to_dev

pytestmark = pytest.mark.gpu


def _run(wl, layout, label, want_lse=True, lists_dev=None):
    import torch
    from packed_varlen_flash_amd import block_layout_csr, pfa_varlen_fwd_blocksparse
    kv_ptr, kv_idx, lh = block_layout_csr(layout, wl.lengths, wl.max_seqlen)
    say(f"[gpu] pfa_varlen_fwd_blocksparse {label}: segs={wl.num_seqs} T={wl.total_tokens} "
        f"H={wl.heads} d={wl.head_dim} layout_heads={lh} nnz={kv_idx.shape[0]}")
    cu = torch.from_numpy(wl.cu_seqlens).to("cuda")
    p = torch.from_numpy(kv_ptr).to("cuda")
    i = torch.from_numpy(kv_idx).to("cuda")
    out, lse = pfa_varlen_fwd_blocksparse(to_dev(wl.q), to_dev(wl.k), to_dev(wl.v), cu, wl.max_seqlen,
                                          p, i, lh, wl.scale, want_lse=want_lse)
    torch.cuda.synchronize()
    return from_dev_bf16(out), (lse.cpu().numpy() if lse is not None else None)


def _check(wl, layout, label, rows=None):
    ob, lse = _run(wl, layout, label)
    o_ref, l_ref = oracle.varlen_fwd_blocksparse(wl.q, wl.k, wl.v, wl.cu_seqlens, wl.scale, layout,
                                                 rows=rows)
    if rows is not None:
        ob, lse = ob[rows], lse[:, rows]
    empty = np.isneginf(l_ref)                       # rows whose list retains no key
    o = W.bf16_to_f64(ob)
    assert np.all(o[empty.T] == 0.0), "rows without keys must be exactly zero"
    assert np.all(np.isneginf(lse[empty])), "rows without keys must have LSE = -inf"
    m = compare(ob, np.where(empty, 0.0, lse).astype(np.float32), o_ref, np.where(empty, 0.0, l_ref))
    assert_parity(m, label)
    return ob, lse


def _pack(seed, d, max_len=1500):
    rng = np.random.default_rng(seed)
    lengths = W.random_lengths(rng, int(rng.integers(1, 7)), max_len)
    if sum(lengths) == 0:
        lengths[0] = 1
    return W.make(lengths, 3, d, seed=seed, name=f"sparse{seed}"), rng


@pytest.mark.parametrize("seed", range(6))
def test_random_layouts_full(seed):
    wl, rng = _pack(300 + seed, 64 if seed % 2 else 128)
    lay = W.random_layout(rng, wl.lengths, wl.heads if seed % 3 == 0 else 1, density=0.5)
    # out-of-range entries are skipped, as the oracle skips them
    lay[0][0] = [row + [-3, 10**6] for row in lay[0][0]]
    _check(wl, lay, f"random layout seed={seed} L={wl.lengths}")


def test_band_layout_c3_sampled():
    wl = W.generate("C3")
    lay = W.band_layout(wl.lengths, radius=1024)
    rows = W.sample_rows(wl.cu_seqlens, stride=61, edge=64, full_upto=0)
    _check(wl, lay, f"C3 band +-1024, sampled {len(rows)} rows", rows=rows)


def test_long_segment_band_sampled():
    wl = W.make([16384, 700], 4, 128, seed=310)
    lay = W.band_layout(wl.lengths, radius=2048)
    rows = W.sample_rows(wl.cu_seqlens, stride=97, edge=64, full_upto=0)
    _check(wl, lay, "16384 + 700 band +-2048", rows=rows)


def test_every_block_listed_equals_the_dense_kernel_bitwise():
    import torch
    from packed_varlen_flash_amd import pfa_varlen_fwd
    wl = W.make([1024, 300, 1, 0, 4096, 65], 3, 128, seed=311)
    full = [[[list(range(-(-L // 64))) for _ in range(-(-L // 256))] for L in wl.lengths]]
    ob, lse = _run(wl, full, "every block listed")
    cu = torch.from_numpy(wl.cu_seqlens).to("cuda")
    out2, lse2 = pfa_varlen_fwd(to_dev(wl.q), to_dev(wl.k), to_dev(wl.v), cu, wl.max_seqlen, wl.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ob, from_dev_bf16(out2))
    np.testing.assert_array_equal(lse, lse2.cpu().numpy())


def test_beyond_the_sort_capacity_every_block_listed_equals_dense_bitwise():
    """4,200 segments, more than the on-device sort holds (4,096): both kernels walk the
    slots (segment, head, tile) in index order, the block-sparse one tile-major.  With every
    block listed the results equal the dense kernel's bit for bit."""
    import torch
    from packed_varlen_flash_amd import pfa_varlen_fwd
    rng = np.random.default_rng(317)
    lengths = [int(x) for x in rng.integers(0, 301, size=4200)]
    lengths[0] = 300                                   # the streaming dense kernel (> 256 keys)
    wl = W.make(lengths, 2, 128, seed=317, name="4200 segments")
    full = [[[list(range(-(-L // 64))) for _ in range(-(-L // 256))] for L in wl.lengths]]
    ob, lse = _run(wl, full, "4200 segments, every block listed")
    cu = torch.from_numpy(wl.cu_seqlens).to("cuda")
    out2, lse2 = pfa_varlen_fwd(to_dev(wl.q), to_dev(wl.k), to_dev(wl.v), cu, wl.max_seqlen, wl.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ob, from_dev_bf16(out2))
    np.testing.assert_array_equal(lse, lse2.cpu().numpy())


def test_list_order_does_not_change_the_retained_set():
    wl, rng = _pack(312, 128)
    lay = W.random_layout(rng, wl.lengths, 1, density=0.6)
    ob, lse = _check(wl, lay, "ascending lists")
    rev = [[[sorted(r, reverse=True) for r in seg] for seg in lay[0]]]
    ob2, lse2 = _check(wl, rev, "descending lists")
    # same keys, other accumulation order: both are within the bars; LSE agrees closely
    np.testing.assert_allclose(lse2[np.isfinite(lse2)], lse[np.isfinite(lse)], rtol=0, atol=1e-4)


def test_empty_layout_and_empty_rows():
    wl = W.make([500, 37], 2, 64, seed=313)
    none = [[[[] for _ in range(-(-L // 256))] for L in wl.lengths]]
    ob, lse = _run(wl, none, "no blocks at all")
    assert np.all(W.bf16_to_f64(ob) == 0.0) and np.all(np.isneginf(lse))
    some = [[[[0, 1], []], [[0]]]]
    _check(wl, some, "one empty query block")


def test_determinism_and_binding_checks():
    import torch
    from packed_varlen_flash_amd import block_layout_csr, pfa_varlen_fwd_blocksparse
    wl = W.make([900, 260], 2, 128, seed=314)
    lay = W.band_layout(wl.lengths, radius=300)
    a = _run(wl, lay, "determinism run 1")
    b = _run(wl, lay, "determinism run 2")
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    kv_ptr, kv_idx, _ = block_layout_csr(lay, wl.lengths, wl.max_seqlen)
    q = to_dev(wl.q)
    cu = torch.from_numpy(wl.cu_seqlens).to("cuda")
    p = torch.from_numpy(kv_ptr[:-1]).to("cuda")           # one row short
    i = torch.from_numpy(kv_idx).to("cuda")
    with pytest.raises(ValueError):
        pfa_varlen_fwd_blocksparse(q, q, q, cu, wl.max_seqlen, p, i)


def test_many_segments_bitonic_schedule():
    # over 512 segments the schedule is sorted by a bitonic network (capacity 1024 here)
    rng = np.random.default_rng(315)
    lengths = [int(x) for x in rng.integers(0, 300, size=700)]
    wl = W.make(lengths, 2, 128, seed=315, name="700 segments")
    lay = W.random_layout(rng, wl.lengths, 1, density=0.7)
    _check(wl, lay, "700 segments, bitonic schedule")


def test_poison_in_other_segments_does_not_leak():
    wl = W.make([300, 700, 90], 2, 128, seed=316)
    lay = W.band_layout(wl.lengths, radius=200)
    ob, lse = _run(wl, lay, "clean")
    a, b = int(wl.cu_seqlens[1]), int(wl.cu_seqlens[2])
    q, k, v = wl.q.copy(), wl.k.copy(), wl.v.copy()
    for arr, val in ((q, 0x7FC0), (k, 0x7F80), (v, 0x7FC0)):
        arr[:a] = val
        arr[b:] = val
    w2 = dataclasses.replace(wl, q=q, k=k, v=v)
    ob2, lse2 = _run(w2, lay, "poisoned neighbours")
    np.testing.assert_array_equal(ob2[a:b], ob[a:b])
    np.testing.assert_array_equal(lse2[:, a:b], lse[:, a:b])
