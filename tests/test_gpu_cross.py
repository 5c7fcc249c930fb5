"""GPU parity of the separate-table forward (pfa_varlen_fwd_qk) and of the (O, LSE) merge
(pfa_attn_merge) against the fp64 oracle, through the C ABI."""
import dataclasses

import numpy as np
import pytest

import oracle
import pfa_workloads as W
from tests._gpu import LSE_ABS, assert_parity, bf16_half_ulp, compare, from_dev_bf16, say, to_dev

pytestmark = pytest.mark.gpu


def _upload(x):
    import torch
    return (to_dev(x.q), to_dev(x.k), to_dev(x.v), torch.from_numpy(x.cu_q).to("cuda"),
            torch.from_numpy(x.cu_k).to("cuda"))


def _run(x, label, dev=None):
    import torch
    from packed_varlen_flash_amd import pfa_varlen_fwd_qk
    say(f"[gpu] pfa_varlen_fwd_qk {label}: segs={x.num_seqs} Tq={x.total_q} Tk={x.total_k} "
        f"H={x.heads} d={x.head_dim}")
    q, k, v, cq, ck = dev if dev is not None else _upload(x)
    out, lse = pfa_varlen_fwd_qk(q, k, v, cq, ck, x.max_q, x.max_k, x.scale)
    torch.cuda.synchronize()
    return from_dev_bf16(out), lse.cpu().numpy()


def _check(x, label, rows=None):
    ob, lse = _run(x, label)
    o_ref, l_ref = oracle.varlen_fwd_qk(x.q, x.k, x.v, x.cu_q, x.cu_k, x.scale, rows=rows)
    if rows is not None:
        ob, lse = ob[rows], lse[:, rows]
    empty = np.isneginf(l_ref)                     # queries whose segment has no keys
    o = W.bf16_to_f64(ob)
    assert np.all(o[empty.T] == 0.0), "rows without keys must be exactly zero"
    assert np.all(np.isneginf(lse[empty])), "rows without keys must have LSE = -inf"
    l_cmp = np.where(empty, 0.0, lse.astype(np.float64))
    m = compare(ob, l_cmp.astype(np.float32), o_ref, np.where(empty, 0.0, l_ref))
    assert_parity(m, label)


def _rect(seed, d):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    lq = W.random_lengths(rng, n, 600)
    lk = W.random_lengths(rng, n, 600)
    if sum(lq) == 0:
        lq[0] = 1
    return W.make_cross(lq, lk, 3, d, seed=seed, name=f"rect{seed}")


@pytest.mark.parametrize("seed", range(8))
def test_random_rectangular_packs_full(seed):
    x = _rect(seed, 64 if seed % 2 else 128)
    _check(x, f"rect seed={seed} Lq={x.lengths_q} Lk={x.lengths_k}")


def test_long_queries_short_keys_full():
    x = W.make_cross([1024, 1296, 4096, 65], [77, 256, 13, 1], 4, 128, seed=11, name="longq")
    _check(x, "long Q, short KV")


def test_short_queries_long_keys_full():
    x = W.make_cross([5, 64, 1, 300], [4096, 2000, 65, 0], 2, 128, seed=12, name="longk")
    _check(x, "short Q, long KV (one empty key segment)")


def test_cross_workload_x1_sampled():
    x = W.generate_cross("X1")
    rows = W.sample_rows(x.cu_q, stride=61, edge=64, full_upto=0)
    _check(x, f"X1 sampled {len(rows)} rows", rows=rows)


def test_equal_tables_match_the_self_attention_kernel_bitwise():
    import torch
    from packed_varlen_flash_amd import pfa_varlen_fwd
    wl = W.make([300, 1, 0, 517, 64], 3, 128, seed=13)
    x = W.make_cross(wl.lengths, wl.lengths, 3, 128, seed=13)
    assert np.array_equal(x.q, wl.q) and np.array_equal(x.k, wl.k)
    q, k, v, cq, ck = _upload(x)          # two distinct device copies of one table
    say("[gpu] equal tables: pfa_varlen_fwd_qk (cross kernel) vs pfa_varlen_fwd")
    o1, l1 = _run(x, "equal tables", dev=(q, k, v, cq, ck))
    o2, l2 = pfa_varlen_fwd(q, k, v, cq, wl.max_seqlen, wl.scale)
    torch.cuda.synchronize()
    assert np.array_equal(o1, from_dev_bf16(o2))
    assert np.array_equal(l1, l2.cpu().numpy())


# ------------------------------------------------------------------------- merge

def _merge_dev(o_a, l_a, o_b, l_b, in_place=False):
    import torch
    from packed_varlen_flash_amd import pfa_attn_merge
    oa, ob = to_dev(o_a), to_dev(o_b)
    la = torch.from_numpy(np.ascontiguousarray(l_a, dtype=np.float32)).to("cuda")
    lb = torch.from_numpy(np.ascontiguousarray(l_b, dtype=np.float32)).to("cuda")
    if in_place:
        out, lse = pfa_attn_merge(oa, la, ob, lb, out=oa, lse=la)
    else:
        out, lse = pfa_attn_merge(oa, la, ob, lb)
    torch.cuda.synchronize()
    return from_dev_bf16(out), lse.cpu().numpy()


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_merge_matches_the_exact_merge_of_its_inputs(d, in_place):
    # Exact reference: the oracle's fp64 merge of the same bf16 / fp32 inputs.  The kernel
    # rounds once to bf16 (at most half the bf16 spacing at |ref|, i.e. <= 2^-8 |ref|) after
    # fp32 arithmetic (relative error a few 2^-24 of |o_a| + |o_b|); LSE is fp32 throughout.
    rng = np.random.default_rng(20 + d)
    T, H = 777, 5
    o_a = W.bf16_bits(rng.standard_normal((T, H, d), dtype=np.float32) * 3)
    o_b = W.bf16_bits(rng.standard_normal((T, H, d), dtype=np.float32) * 3)
    l_a = (rng.standard_normal((H, T)) * 4).astype(np.float32)
    l_b = (rng.standard_normal((H, T)) * 4).astype(np.float32)
    l_b[:, ::7] = -np.inf                       # B empty for some rows
    l_a[:, ::11] = -np.inf                      # A empty for others (both for some)
    say(f"[gpu] pfa_attn_merge d={d} in_place={in_place} T={T} H={H}")
    out, lse = _merge_dev(o_a, l_a, o_b, l_b, in_place)
    fa, fb = W.bf16_to_f64(o_a), W.bf16_to_f64(o_b)
    o_ref, l_ref = oracle.merge(fa, l_a.astype(np.float64), fb, l_b.astype(np.float64))
    o = W.bf16_to_f64(out)
    bound = bf16_half_ulp(o_ref) + 2.0 ** -20 * (np.abs(fa) + np.abs(fb)) + 1e-38
    assert np.all(np.abs(o - o_ref) <= bound)
    both = np.isneginf(l_ref)
    assert np.all(np.isneginf(lse[both])) and np.all(o[both.T] == 0.0)
    assert np.all(np.abs(lse[~both] - l_ref[~both]) <= 1e-6 * (1.0 + np.abs(l_ref[~both])))


def test_merge_of_two_key_halves_end_to_end():
    # Each segment's keys split in two; forward on each half, merge, compare with the
    # oracle over the whole segment.  Tolerance: the forward bars, except that the two
    # partial outputs are each rounded to bf16 before merging, which adds at most
    # 2^-8 max|O| to max|err| and at most 2^-8/sqrt(3) to the relative RMS (the RMS of
    # a rounding error spread uniformly within half a bf16 spacing).
    import torch
    from packed_varlen_flash_amd import pfa_attn_merge, pfa_varlen_fwd_qk
    lq, la, lb = [700, 1296, 64], [500, 1, 2000], [300, 900, 0]
    H, d, seed = 4, 128, 31
    full = W.make_cross(lq, [a + b for a, b in zip(la, lb)], H, d, seed=seed, name="union")
    ka, kb, va, vb = [], [], [], []
    for s in range(3):
        a0 = int(full.cu_k[s])
        ka.append(full.k[a0:a0 + la[s]]); kb.append(full.k[a0 + la[s]:a0 + la[s] + lb[s]])
        va.append(full.v[a0:a0 + la[s]]); vb.append(full.v[a0 + la[s]:a0 + la[s] + lb[s]])
    cat = lambda parts: np.ascontiguousarray(np.concatenate(parts, axis=0))
    q = to_dev(full.q)
    cu_q = torch.from_numpy(full.cu_q).to("cuda")
    outs = []
    for kk, vv, lens in ((cat(ka), cat(va), la), (cat(kb), cat(vb), lb)):
        cu_k = torch.from_numpy(W.cu_from_lengths(lens)).to("cuda")
        say(f"[gpu] merge end-to-end: pfa_varlen_fwd_qk on key lengths {lens}")
        outs.append(pfa_varlen_fwd_qk(q, to_dev(kk), to_dev(vv), cu_q, cu_k, max(lq),
                                      max(max(lens), 1), full.scale))
    say("[gpu] merge end-to-end: pfa_attn_merge")
    out, lse = pfa_attn_merge(outs[0][0], outs[0][1], outs[1][0], outs[1][1])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.varlen_fwd_qk(full.q, full.k, full.v, full.cu_q, full.cu_k, full.scale)
    m = compare(from_dev_bf16(out), lse.cpu().numpy(), o_ref, l_ref)
    extra = 2.0 ** -8 * float(np.abs(o_ref).max())
    say(f"[parity] merge end-to-end: max|err|={m['max_abs']:.3e} relRMS={m['rel_rms']:.3e} "
        f"LSE={m['lse_abs']:.3e} (allowance for the partials' rounding {extra:.3e})")
    assert m["max_abs_small"] <= 1e-2 + extra
    assert m["rel_rms"] <= 4e-3 + 2.0 ** -8 / np.sqrt(3.0)
    assert m["lse_abs"] <= LSE_ABS


def test_poison_in_other_segments_does_not_leak():
    # NaN / Inf in the rows of other segments (queries and keys) leave segment 1 bitwise equal
    x = W.make_cross([300, 257, 40], [90, 513, 7], 2, 128, seed=14, name="poison")
    ob, lse = _run(x, "clean")
    q, k, v = x.q.copy(), x.k.copy(), x.v.copy()
    qa, qb = int(x.cu_q[1]), int(x.cu_q[2])
    ka, kb = int(x.cu_k[1]), int(x.cu_k[2])
    q[:qa] = q[qb:] = 0x7FC0
    k[:ka] = k[kb:] = 0x7F80
    v[:ka] = v[kb:] = 0x7FC0
    y = dataclasses.replace(x, q=q, k=k, v=v)
    ob2, lse2 = _run(y, "poisoned neighbours")
    np.testing.assert_array_equal(ob2[qa:qb], ob[qa:qb])
    np.testing.assert_array_equal(lse2[:, qa:qb], lse[:, qa:qb])


# ---- short key segments: the resident-K/V kernel (every key segment held in LDS for all
# of its query tiles; chosen when max_seqlen_k <= 256 at d = 128, <= 128 at d = 64)

def _short_keys(seed, d, kmax):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 7))
    lq = [int(x) for x in rng.integers(1, 1800, size=n)]
    lk = W.random_lengths(rng, n, kmax)
    return W.make_cross(lq, lk, 3, d, seed=seed, name=f"shortk{seed}")


@pytest.mark.parametrize("seed", range(6))
def test_resident_kv_random_packs_full(seed):
    d = 64 if seed % 2 else 128
    x = _short_keys(500 + seed, d, 128 if d == 64 else 256)   # max_k = longest key segment
    _check(x, f"resident K/V seed={seed} d={d} Lq={x.lengths_q} Lk={x.lengths_k}")


def test_resident_kv_matches_the_streaming_kernel_bitwise():
    """The same data through both kernels (a key bound above the resident limit selects
    the streaming one): same stages in the same order, so bitwise equal."""
    import torch
    from packed_varlen_flash_amd import pfa_varlen_fwd_qk
    for d, kmax in ((128, 256), (64, 128)):
        x = W.make_cross([4096, 1, 300, 1024, 700, 0], [256, 1, 64, 0, 200, 5] if d == 128 else
                         [128, 1, 64, 0, 100, 5], 4, d, seed=600 + d, name="resident-vs-stream")
        q, k, v, cq, ck = _upload(x)
        o1, l1 = pfa_varlen_fwd_qk(q, k, v, cq, ck, x.max_q, kmax, x.scale)        # resident
        o2, l2 = pfa_varlen_fwd_qk(q, k, v, cq, ck, x.max_q, kmax + 1, x.scale)    # streaming
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), d
        assert torch.equal(l1, l2), d


@pytest.mark.parametrize("d", [128, 64])
def test_resident_kv_switching_matches_the_streaming_kernel_bitwise(d):
    """More tiles than workgroups, so each workgroup runs several (segment, head) key sets in
    a row and loads the next one into the slots of the last tile as it frees them: key
    stage counts rising, falling, and an empty key segment between them."""
    import torch
    from packed_varlen_flash_amd import pfa_varlen_fwd_qk
    kmax = 256 if d == 128 else 128
    lk = [256, 0, 64, 200, 1, 130] if d == 128 else [128, 0, 64, 100, 1, 65]
    heads = 32 if d == 128 else 48
    x = W.make_cross([2048, 1500, 700, 3000, 1, 900], lk, heads, d, seed=700 + d, name="resident-switch")
    q, k, v, cq, ck = _upload(x)
    say(f"[gpu] resident K/V switching d={d} H={heads} Lk={lk}")
    o1, l1 = pfa_varlen_fwd_qk(q, k, v, cq, ck, x.max_q, kmax, x.scale)        # resident
    o2, l2 = pfa_varlen_fwd_qk(q, k, v, cq, ck, x.max_q, kmax + 1, x.scale)    # streaming
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), d
    assert torch.equal(l1, l2), d
    # and the resident kernel against the oracle on sampled rows of every segment
    rows = W.sample_rows(x.cu_q, stride=97, edge=8, full_upto=0)
    _check(x, f"resident-switch d={d} sampled {len(rows)} rows", rows=rows)


@pytest.mark.parametrize("n,d", [(600, 128), (700, 64), (4200, 128)])
def test_many_segments_resident_and_streaming_schedules(n, d):
    """Over 512 segments the resident kernel walks the unsorted slots while the streaming
    kernel sorts them (bitonic, up to 4,096) or also walks them (4,200): every tile is
    computed once whatever the order, so the two kernels agree bitwise, and a sample of rows
    against the oracle."""
    import torch
    from packed_varlen_flash_amd import pfa_varlen_fwd_qk
    kmax = 256 if d == 128 else 128
    rng = np.random.default_rng(800 + n)
    lq = [int(x) for x in rng.integers(0, 300, size=n)]
    lk = [int(x) for x in rng.integers(0, kmax + 1, size=n)]
    lq[int(rng.integers(0, n))] = 1500                # one multi-tile query segment
    x = W.make_cross(lq, lk, 2, d, seed=800 + n, name=f"{n} cross segments")
    q, k, v, cq, ck = _upload(x)
    say(f"[gpu] {n} cross segments d={d}: resident (unsorted) vs streaming")
    o1, l1 = pfa_varlen_fwd_qk(q, k, v, cq, ck, x.max_q, kmax, x.scale)        # resident
    o2, l2 = pfa_varlen_fwd_qk(q, k, v, cq, ck, x.max_q, kmax + 1, x.scale)    # streaming
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    rows = W.sample_rows(x.cu_q, stride=53, edge=4, full_upto=0)
    _check(x, f"{n} cross segments d={d} sampled {len(rows)} rows", rows=rows)
