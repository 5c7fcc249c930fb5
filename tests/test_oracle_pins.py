"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test names the passage it follows.  None compares the oracle with a retyped copy
of its own formula: the pins are printed values (SparseAttn worked example), closed
forms, a dense masked brute force, PyTorch's own attention routine, and invariants.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import pfa_workloads as W
from tests._brute import dense_block_diag

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sparseattn_worked_example.json")


def _printed_tol(s: str) -> float:
    """Half a unit in the last printed digit (values on the page are rounded)."""
    mant = s.lower().split("e")[0]
    exp = int(s.lower().split("e")[1]) if "e" in s.lower() else 0
    decimals = len(mant.split(".")[1]) if "." in mant else 0
    return 0.5 * 10.0 ** (exp - decimals) * 1.001


# ------------------------------------------------------------------ P-e worked example

@pytest.fixture(scope="module")
def worked():
    ex = W.worked_example()
    q = np.ascontiguousarray(ex.q.transpose(1, 0, 2))            # [64, 2, 20]
    v = np.ascontiguousarray(np.repeat(ex.v[:, None, :], 2, 1))  # [64, 2, 3], shared by heads
    scale = 1.0 / math.sqrt(q.shape[2])
    n = q.shape[0]
    full_o, full_l = oracle.varlen_fwd(q, q, v, [0, n], scale)
    # same-frame mask == pack of the 4 frames (tokens are frame-major)
    sf_o, sf_l = oracle.varlen_fwd(q, q, v, list(range(0, n + 1, ex.positions)), scale)
    # same-position mask == pack of 16 groups of 4 after a stable sort by position
    perm = np.argsort(ex.pixel, kind="stable")
    inv = np.empty_like(perm)
    inv[perm] = np.arange(n)
    sp_o, sp_l = oracle.varlen_fwd(q[perm], q[perm], v[perm], list(range(0, n + 1, ex.frames)), scale)
    sp_o, sp_l = sp_o[inv], sp_l[:, inv]
    with open(GOLDEN) as f:
        gold = json.load(f)["values"]
    return dict(v=ex.v, full=(full_o, full_l), sf=(sf_o, sf_l), sp=(sp_o, sp_l), gold=gold)


def _check(gold, key, value):
    want = float(gold[key])
    assert abs(value - want) <= _printed_tol(gold[key]), (key, value, want)


@pytest.mark.parametrize("head,mask,prefix", [
    (0, "sf", "spatial_head_same_frame"),
    (0, "sp", "spatial_head_same_position"),
    (1, "sf", "temporal_head_same_frame"),
    (1, "sp", "temporal_head_same_position"),
])
def test_worked_example_retained_mass_and_mse(worked, head, mask, prefix):
    """SparseAttn article, section 04 table: retained mass and MSE vs full attention."""
    full_o, full_l = worked["full"]
    o, l = worked[mask]
    retained = np.exp(l[head] - full_l[head])          # z_i = sum_{j in S_i} p_ij (section 3.1)
    mse = float(np.mean((o[:, head, :] - full_o[:, head, :]) ** 2))
    _check(worked["gold"], prefix + "_retained_mass", float(retained.mean()))
    _check(worked["gold"], prefix + "_mse", mse)


def test_worked_example_row_error_and_bound(worked):
    """SparseAttn article, sections 3.2 and 04: per-row error <= 2*alpha_i*M, printed maxima."""
    full_o, full_l = worked["full"]
    o, l = worked["sf"]
    alpha = 1.0 - np.exp(l[0] - full_l[0])
    err = np.linalg.norm(o[:, 0, :] - full_o[:, 0, :], axis=1)
    M = np.linalg.norm(worked["v"], axis=1).max()
    bound = 2.0 * np.maximum(alpha, 0.0) * M
    assert np.all(err <= bound + 1e-12)
    _check(worked["gold"], "spatial_head_same_frame_max_row_error", float(err.max()))
    _check(worked["gold"], "spatial_head_same_frame_max_bound", float(bound.max()))


def test_worked_example_full_mask_is_exact(worked):
    """Section 04: the same inputs under the full mask reproduce full attention exactly."""
    ex = W.worked_example()
    q = np.ascontiguousarray(ex.q.transpose(1, 0, 2))
    v = np.ascontiguousarray(np.repeat(ex.v[:, None, :], 2, 1))
    o, l = oracle.varlen_fwd(q, q, v, [0, 64], 1.0 / math.sqrt(20))
    assert np.array_equal(o, worked["full"][0]) and np.array_equal(l, worked["full"][1])


# --------------------------------------------------------------------- P-f closed forms

def test_single_token_segment_returns_its_value():
    """L = 1: the only weight is 1, so O = v exactly and LSE = scale * q.k."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((5, 3, 8)); k = rng.standard_normal((5, 3, 8))
    v = rng.standard_normal((5, 3, 4))
    cu = [0, 2, 3, 5]                                   # token 2 is alone
    o, l = oracle.varlen_fwd(q, k, v, cu, 0.7)
    assert np.array_equal(o[2], v[2])
    np.testing.assert_allclose(l[:, 2], 0.7 * np.sum(q[2] * k[2], axis=1), rtol=0, atol=1e-14)


def test_zero_queries_give_segment_mean():
    """q = 0 in a segment: uniform weights, O = mean of the segment's V, LSE = ln L."""
    rng = np.random.default_rng(4)
    T, H, d = 12, 2, 6
    q = rng.standard_normal((T, H, d)); k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, 5))
    q[4:11] = 0.0
    cu = [0, 4, 11, 12]
    o, l = oracle.varlen_fwd(q, k, v, cu, 0.3)
    np.testing.assert_allclose(o[4:11], np.broadcast_to(v[4:11].mean(axis=0), (7, H, 5)), atol=1e-14)
    np.testing.assert_allclose(l[:, 4:11], math.log(7), atol=1e-14)


def test_constant_values_are_reproduced():
    """V equal to c across a segment: any convex combination returns c."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((9, 1, 4)); k = rng.standard_normal((9, 1, 4))
    v = rng.standard_normal((9, 1, 3)); v[3:9] = np.array([1.5, -2.0, 0.25])
    o, _ = oracle.varlen_fwd(q, k, v, [0, 3, 9], 1.0)
    np.testing.assert_allclose(o[3:9, 0], np.broadcast_to([1.5, -2.0, 0.25], (6, 3)), atol=1e-14)


def test_two_key_counterexample():
    """SparseAttn article, section 3.2: query 1, keys ln 99 and 0, values 0 and 100 give
    probabilities 0.99/0.01 and output 1; keeping only the first key gives output 0."""
    q = np.array([[[1.0]], [[1.0]]]); k = np.array([[[math.log(99.0)]], [[0.0]]])
    v = np.array([[[0.0]], [[100.0]]])
    o, l = oracle.varlen_fwd(q, k, v, [0, 2], 1.0)
    np.testing.assert_allclose(o[:, 0, 0], [1.0, 1.0], atol=1e-12)
    np.testing.assert_allclose(l[0], [math.log(100.0)] * 2, atol=1e-14)
    p = oracle.probs(q, k, [0, 2], 1.0, 0, 0)
    np.testing.assert_allclose(p, [0.99, 0.01], atol=1e-15)
    o1, _ = oracle.varlen_fwd(q[:1], k[:1], v[:1], [0, 1], 1.0)      # retained set {key 0}
    assert o1[0, 0, 0] == 0.0


def test_large_logits_do_not_overflow():
    """Logits near 1000: p = (3/4, 1/4) and LSE = 1000 + ln(4/3); a softmax that does not
    subtract the row maximum overflows here."""
    q = np.ones((2, 1, 1)); k = np.array([[[1000.0]], [[1000.0 - math.log(3.0)]]])
    v = np.array([[[0.0]], [[4.0]]])
    o, l = oracle.varlen_fwd(q, k, v, [0, 2], 1.0)
    np.testing.assert_allclose(o[:, 0, 0], [1.0, 1.0], atol=1e-12)
    np.testing.assert_allclose(l[0], 1000.0 + math.log(4.0 / 3.0), atol=1e-12)


# -------------------------------------------------------- P-a brute force, P-h library

def _random_case(seed, max_segs=7, max_len=40, H=3, d=16, dv=None, bf16=False):
    rng = np.random.default_rng(seed)
    lengths = W.random_lengths(rng, int(rng.integers(1, max_segs + 1)), max_len)
    if sum(lengths) == 0:
        lengths[0] = 1
    T = sum(lengths)
    dv = dv or d
    q = rng.standard_normal((T, H, d)); k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, dv))
    if bf16:
        q, k, v = W.bf16_bits(q), W.bf16_bits(k), W.bf16_bits(v)
    return lengths, W.cu_from_lengths(lengths), q, k, v


@pytest.mark.parametrize("seed", range(12))
def test_matches_dense_brute_force(seed):
    """Dense masked T x T softmax (GigaPath-Flash 4.1 naive form + SparseAttn -inf mask)."""
    lengths, cu, q, k, v = _random_case(seed, dv=[16, 5, 16][seed % 3], bf16=seed % 2 == 1)
    scale = 0.25 + 0.1 * seed
    o, l = oracle.varlen_fwd(q, k, v, cu, scale)
    qf, kf, vf = (W.bf16_to_f64(x) if x.dtype == np.uint16 else x for x in (q, k, v))
    ob, lb = dense_block_diag(qf, kf, vf, cu, scale)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_matches_torch_sdpa_fp64(seed):
    """PyTorch's scaled_dot_product_attention (fp64, CPU, non-causal) run per segment,
    and torch.logsumexp of the scaled scores for the LSE (GigaPath-Flash 4.3 names SDPA)."""
    lengths, cu, q, k, v = _random_case(100 + seed, H=2, d=32)
    scale = 1.0 / math.sqrt(32)
    o, l = oracle.varlen_fwd(q, k, v, cu, scale)
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        if a == b:
            continue
        qs = torch.from_numpy(q[a:b]).permute(1, 0, 2)[None]
        ks = torch.from_numpy(k[a:b]).permute(1, 0, 2)[None]
        vs = torch.from_numpy(v[a:b]).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, is_causal=False, scale=scale)
        np.testing.assert_allclose(o[a:b], ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        lref = torch.logsumexp(scale * qs[0] @ ks[0].transpose(1, 2), dim=-1)
        np.testing.assert_allclose(l[:, a:b], lref.numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------------------- invariants

def test_probability_rows_sum_to_one_and_vanish_off_segment():
    """Every row of the restricted softmax sums to 1 (SparseAttn section 3.1 renormalisation)
    and assigns nothing outside the query's own segment (Mage-Flow: block-diagonal mask)."""
    lengths, cu, q, k, v = _random_case(7, H=2, d=8)
    T = cu[-1]
    o, _ = oracle.varlen_fwd(q, k, v, cu, 0.5)
    for i in range(0, T, 3):
        s = int(np.searchsorted(cu[1:], i, side="right"))
        for h in range(2):
            p = oracle.probs(q, k, cu, 0.5, i, h)
            assert abs(p.sum() - 1.0) < 1e-14
            assert np.all(p[: cu[s]] == 0) and np.all(p[cu[s + 1]:] == 0)
            np.testing.assert_allclose(p @ v[:, h, :], o[i, h], atol=1e-13)


def test_pack_equals_each_segment_alone():
    """A packed result equals every image run by itself (block-diagonal statement)."""
    lengths, cu, q, k, v = _random_case(8, bf16=True)
    o, l = oracle.varlen_fwd(q, k, v, cu, 0.4)
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        if a == b:
            continue
        os_, ls_ = oracle.varlen_fwd(q[a:b], k[a:b], v[a:b], [0, b - a], 0.4)
        assert np.array_equal(o[a:b], os_) and np.array_equal(l[:, a:b], ls_)


@pytest.mark.parametrize("poison", [np.nan, np.inf, 1e30])
def test_other_segments_cannot_leak(poison):
    """Poisoning every other segment leaves a segment's output bitwise unchanged
    (LinearMem article: packed samples must not leak state; Mage-Flow block mask)."""
    lengths, cu, q, k, v = _random_case(9)
    o, l = oracle.varlen_fwd(q, k, v, cu, 0.5)
    target = max(range(len(lengths)), key=lambda s: lengths[s])
    a, b = int(cu[target]), int(cu[target + 1])
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for arr in (q2, k2, v2):
        arr[:a] = poison
        arr[b:] = poison
    o2, l2 = oracle.varlen_fwd(q2, k2, v2, cu, 0.5)
    assert np.array_equal(o2[a:b], o[a:b]) and np.array_equal(l2[:, a:b], l[:, a:b])


def test_permutation_equivariance():
    """SparseAttn article, section 3.4: permuting tokens consistently (segment order, and
    order inside a segment) permutes the outputs; fp64 differences stay at rounding."""
    lengths, cu, q, k, v = _random_case(10, max_segs=5)
    o, l = oracle.varlen_fwd(q, k, v, cu, 0.5)
    rng = np.random.default_rng(11)
    order = rng.permutation(len(lengths))
    idx = []
    for s in order:
        a, b = int(cu[s]), int(cu[s + 1])
        idx.extend(list(a + rng.permutation(b - a)))
    idx = np.array(idx, dtype=np.int64)
    cu2 = W.cu_from_lengths([lengths[s] for s in order])
    o2, l2 = oracle.varlen_fwd(q[idx], k[idx], v[idx], cu2, 0.5)
    np.testing.assert_allclose(o2, o[idx], rtol=0, atol=4e-15)
    np.testing.assert_allclose(l2, l[:, idx], rtol=0, atol=4e-15)


def test_deletion_mass_bound_between_pack_and_merged_sequence():
    """SparseAttn article, section 3.2: ||O_pack - O_full|| <= 2 alpha_i max||v||, with
    alpha_i = 1 - exp(LSE_pack - LSE_full) the probability mass the pack removes."""
    lengths, cu, q, k, v = _random_case(12, H=2, d=4)
    T = int(cu[-1])
    op, lp = oracle.varlen_fwd(q, k, v, cu, 1.0)
    of, lf = oracle.varlen_fwd(q, k, v, [0, T], 1.0)
    for h in range(2):
        alpha = np.maximum(1.0 - np.exp(lp[h] - lf[h]), 0.0)
        M = np.linalg.norm(v[:, h, :], axis=1).max()
        err = np.linalg.norm(op[:, h, :] - of[:, h, :], axis=1)
        assert np.all(err <= 2 * alpha * M + 1e-12)


def test_row_sample_matches_full_run():
    lengths, cu, q, k, v = _random_case(13, bf16=True)
    o, l = oracle.varlen_fwd(q, k, v, cu, 0.5)
    rows = np.arange(0, int(cu[-1]), 2)
    os_, ls_ = oracle.varlen_fwd(q, k, v, cu, 0.5, rows=rows)
    assert np.array_equal(os_, o[rows]) and np.array_equal(ls_, l[:, rows])


def test_rejects_malformed_tables():
    q = np.zeros((4, 1, 2)); v = np.zeros((4, 1, 2))
    with pytest.raises(ValueError):
        oracle.varlen_fwd(q, q, v, [0, 3, 2, 4], 1.0)      # decreasing
    with pytest.raises(ValueError):
        oracle.varlen_fwd(q, q, v, [1, 4], 1.0)            # does not start at 0


# ---------------------------------------------------------------------------------
# Separate query / key tables (the varlen call's cu_seqlens_q and cu_seqlens_k) and the
# (O, LSE) merge of two disjoint key sets.
# ---------------------------------------------------------------------------------
from tests._brute import dense_block_rect  # noqa: E402


def _rect_case(seed, H=3, d=8, dv=5):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 6))
    lq = rng.integers(0, 9, size=n)
    lk = rng.integers(0, 9, size=n)
    lq[0] = max(lq[0], 1)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = rng.standard_normal((int(cu_q[-1]), H, d))
    k = rng.standard_normal((int(cu_k[-1]), H, d))
    v = rng.standard_normal((int(cu_k[-1]), H, dv))
    return q, k, v, cu_q, cu_k


@pytest.mark.parametrize("seed", range(12))
def test_qk_tables_match_dense_rectangular_brute_force(seed):
    q, k, v, cu_q, cu_k = _rect_case(seed)
    o, l = oracle.varlen_fwd_qk(q, k, v, cu_q, cu_k, 0.4)
    ob, lb = dense_block_rect(q, k, v, cu_q, cu_k, 0.4)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    finite = np.isfinite(lb)
    np.testing.assert_array_equal(np.isfinite(l), finite)
    np.testing.assert_allclose(l[finite], lb[finite], rtol=0, atol=1e-13)


def test_qk_tables_match_torch_sdpa_per_segment():
    rng = np.random.default_rng(3)
    lq, lk = [37, 5, 64], [7, 90, 1]
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = rng.standard_normal((sum(lq), 2, 16))
    k = rng.standard_normal((sum(lk), 2, 16))
    v = rng.standard_normal((sum(lk), 2, 16))
    o, _ = oracle.varlen_fwd_qk(q, k, v, cu_q, cu_k, 0.25)
    for s in range(3):
        qs = torch.from_numpy(q[cu_q[s]:cu_q[s + 1]]).permute(1, 0, 2)
        ks = torch.from_numpy(k[cu_k[s]:cu_k[s + 1]]).permute(1, 0, 2)
        vs = torch.from_numpy(v[cu_k[s]:cu_k[s + 1]]).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, scale=0.25)
        np.testing.assert_allclose(o[cu_q[s]:cu_q[s + 1]], ref.permute(1, 0, 2).numpy(), atol=1e-12)


def test_qk_tables_closed_forms():
    # one key per segment: the output is that key's value and LSE = scale * q.k
    rng = np.random.default_rng(5)
    cu_q = np.array([0, 4, 9], np.int32)
    cu_k = np.array([0, 1, 2], np.int32)
    q = rng.standard_normal((9, 2, 6))
    k = rng.standard_normal((2, 2, 6))
    v = rng.standard_normal((2, 2, 3))
    o, l = oracle.varlen_fwd_qk(q, k, v, cu_q, cu_k, 0.7)
    for i in range(9):
        s = 0 if i < 4 else 1
        np.testing.assert_array_equal(o[i], v[s])
        for h in range(2):
            assert abs(l[h, i] - 0.7 * float(q[i, h] @ k[s, h])) < 1e-14
    # zero queries: uniform weights over the key segment, LSE = ln(Lk)
    q0 = np.zeros((9, 2, 6))
    cu_k2 = np.array([0, 3, 10], np.int32)
    k2 = rng.standard_normal((10, 2, 6))
    v2 = rng.standard_normal((10, 2, 3))
    o, l = oracle.varlen_fwd_qk(q0, k2, v2, cu_q, cu_k2, 1.0)
    np.testing.assert_allclose(o[:4], np.broadcast_to(v2[:3].mean(axis=0), (4, 2, 3)), atol=1e-15)
    np.testing.assert_allclose(o[4:], np.broadcast_to(v2[3:].mean(axis=0), (5, 2, 3)), atol=1e-15)
    np.testing.assert_allclose(l[:, :4], math.log(3), atol=1e-15)
    np.testing.assert_allclose(l[:, 4:], math.log(7), atol=1e-15)


def test_qk_tables_empty_key_segment_gives_zero_and_minus_inf():
    rng = np.random.default_rng(6)
    cu_q = np.array([0, 3, 5], np.int32)
    cu_k = np.array([0, 0, 4], np.int32)
    q = rng.standard_normal((5, 2, 4))
    k = rng.standard_normal((4, 2, 4))
    v = rng.standard_normal((4, 2, 4))
    o, l = oracle.varlen_fwd_qk(q, k, v, cu_q, cu_k, 1.0)
    assert np.all(o[:3] == 0.0) and np.all(np.isneginf(l[:, :3]))
    assert np.all(np.isfinite(l[:, 3:]))


def test_qk_tables_with_equal_tables_equal_self_attention():
    rng = np.random.default_rng(8)
    cu = np.array([0, 5, 5, 17], np.int32)
    q, k, v = (rng.standard_normal((17, 2, 8)) for _ in range(3))
    o1, l1 = oracle.varlen_fwd(q, k, v, cu, 0.3)
    o2, l2 = oracle.varlen_fwd_qk(q, k, v, cu, cu, 0.3)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("seed", range(6))
def test_merge_of_two_key_halves_equals_attention_over_the_union(seed):
    # keys of each segment split into a first and a second part (either may be empty):
    # attention over the whole segment = merge of the attentions over the two parts
    rng = np.random.default_rng(100 + seed)
    n, H, d, dv = 3, 2, 8, 4
    lq = rng.integers(1, 7, size=n)
    la = rng.integers(0, 6, size=n)
    lb = rng.integers(0, 6, size=n)
    lb[la + lb == 0] = 1
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    q = rng.standard_normal((int(cu_q[-1]), H, d))
    ka = [rng.standard_normal((int(x), H, d)) for x in la]
    kb = [rng.standard_normal((int(x), H, d)) for x in lb]
    va = [rng.standard_normal((int(x), H, dv)) for x in la]
    vb = [rng.standard_normal((int(x), H, dv)) for x in lb]
    cat = lambda parts: np.concatenate(parts, axis=0)
    cu_a = np.concatenate([[0], np.cumsum(la)]).astype(np.int32)
    cu_b = np.concatenate([[0], np.cumsum(lb)]).astype(np.int32)
    cu_u = np.concatenate([[0], np.cumsum(la + lb)]).astype(np.int32)
    o_a, l_a = oracle.varlen_fwd_qk(q, cat(ka), cat(va), cu_q, cu_a, 0.5)
    o_b, l_b = oracle.varlen_fwd_qk(q, cat(kb), cat(vb), cu_q, cu_b, 0.5)
    ku = cat([np.concatenate([a, b]) for a, b in zip(ka, kb)])
    vu = cat([np.concatenate([a, b]) for a, b in zip(va, vb)])
    o_u, l_u = oracle.varlen_fwd_qk(q, ku, vu, cu_q, cu_u, 0.5)
    o_m, l_m = oracle.merge(o_a, l_a, o_b, l_b)
    np.testing.assert_allclose(o_m, o_u, atol=1e-13)
    np.testing.assert_allclose(l_m, l_u, atol=1e-13)


def test_merge_special_cases():
    rng = np.random.default_rng(9)
    o_a = rng.standard_normal((4, 2, 3))
    o_b = rng.standard_normal((4, 2, 3))
    l_a = rng.standard_normal((2, 4))
    # an empty side contributes nothing
    o, l = oracle.merge(o_a, l_a, o_b, np.full((2, 4), -np.inf))
    np.testing.assert_array_equal(o, o_a)
    np.testing.assert_array_equal(l, l_a)
    # equal partition sums: the plain mean, LSE + ln 2
    o, l = oracle.merge(o_a, l_a, o_b, l_a)
    np.testing.assert_allclose(o, 0.5 * (o_a + o_b), atol=1e-15)
    np.testing.assert_allclose(l, l_a + math.log(2.0), atol=1e-15)
    # two empty sides: zero output, -inf
    o, l = oracle.merge(o_a, np.full((2, 4), -np.inf), o_b, np.full((2, 4), -np.inf))
    assert np.all(o == 0.0) and np.all(np.isneginf(l))


def test_qk_oracle_rejects_mismatched_tables():
    q = np.zeros((4, 1, 2))
    with pytest.raises(ValueError):
        oracle.varlen_fwd_qk(q, q, q, np.array([0, 4], np.int32), np.array([0, 2, 4], np.int32), 1.0)
    with pytest.raises(ValueError):
        oracle.varlen_fwd_qk(q, q[:3], q[:3], np.array([0, 4], np.int32), np.array([0, 4], np.int32), 1.0)


# ---------------------------------------------------------------------------------
# Backward (dQ, dK, dV for an upstream gradient dO of O).
# ---------------------------------------------------------------------------------

def _bwd_case(seed, lengths=(5, 1, 0, 9), H=2, d=6):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    return [rng.standard_normal((T, H, d)) for _ in range(4)] + [cu]


@pytest.mark.parametrize("seed", range(4))
def test_backward_matches_finite_differences_of_the_forward(seed):
    # f = sum(dO * O(q, k, v)); its directional derivative along a random direction must
    # equal <grad, direction>.  Central differences of the fp64 forward oracle, step 1e-5:
    # truncation ~1e-10, cancellation ~1e-11.
    q, k, v, do, cu = _bwd_case(seed)
    scale = 0.7
    dq, dk, dv = oracle.varlen_bwd(q, k, v, do, cu, scale)
    rng = np.random.default_rng(100 + seed)
    f = lambda a, b, c: float((oracle.varlen_fwd(a, b, c, cu, scale)[0] * do).sum())
    eps = 1e-5
    for which in range(3):
        dirs = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)]
        dirs[which] = rng.standard_normal(q.shape)
        plus = [x + eps * e for x, e in zip((q, k, v), dirs)]
        minus = [x - eps * e for x, e in zip((q, k, v), dirs)]
        fd = (f(*plus) - f(*minus)) / (2 * eps)
        an = float(((dq, dk, dv)[which] * dirs[which]).sum())
        assert abs(fd - an) <= 1e-7 * (1.0 + abs(an)), (which, fd, an)


def test_backward_matches_torch_autograd_fp64():
    q, k, v, do, cu = _bwd_case(7, lengths=(33, 2, 17), H=3, d=16)
    scale = 0.25
    dq, dk, dv = oracle.varlen_bwd(q, k, v, do, cu, scale)
    for s in range(3):
        sl = slice(int(cu[s]), int(cu[s + 1]))
        tq, tk, tv = (torch.tensor(x[sl].transpose(1, 0, 2), requires_grad=True) for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
        o.backward(torch.tensor(do[sl].transpose(1, 0, 2)))
        for ours, ref in ((dq, tq), (dk, tk), (dv, tv)):
            np.testing.assert_allclose(ours[sl], ref.grad.numpy().transpose(1, 0, 2), atol=1e-12)


def test_backward_closed_forms():
    # length 1: the softmax weight is 1 whatever the score, so dQ = dK = 0 and dV = dO
    q, k, v, do, cu = _bwd_case(3, lengths=(1, 1, 1), H=2, d=5)
    dq, dk, dv = oracle.varlen_bwd(q, k, v, do, cu, 0.9)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    np.testing.assert_array_equal(dv, do)
    # values constant over a segment: O does not depend on the weights, so dQ = dK = 0,
    # and dV_j = sum_i P_ij dO_i sums (over keys) to the segment's total dO
    q, k, v, do, cu = _bwd_case(4, lengths=(6, 4), H=1, d=3)
    v[:6] = 1.5
    v[6:] = -2.0
    dq, dk, dv = oracle.varlen_bwd(q, k, v, do, cu, 1.1)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    np.testing.assert_allclose(dv[:6].sum(axis=0), do[:6].sum(axis=0), atol=1e-13)
    np.testing.assert_allclose(dv[6:].sum(axis=0), do[6:].sum(axis=0), atol=1e-13)


def test_backward_key_gradients_sum_to_zero_per_segment():
    # every row of dS sums to zero (softmax Jacobian), so sum_j dK_j = scale sum_i q_i
    # sum_j dS_ij = 0 within each segment and head
    q, k, v, do, cu = _bwd_case(5, lengths=(40, 3, 17), H=2, d=8)
    _, dk, _ = oracle.varlen_bwd(q, k, v, do, cu, 0.6)
    for s in range(3):
        tot = dk[cu[s]:cu[s + 1]].sum(axis=0)
        np.testing.assert_allclose(tot, 0.0, atol=1e-12)


def test_backward_pack_equals_each_segment_alone():
    q, k, v, do, cu = _bwd_case(6, lengths=(7, 0, 12, 3), H=2, d=4)
    full = oracle.varlen_bwd(q, k, v, do, cu, 0.5)
    for s in range(4):
        sl = slice(int(cu[s]), int(cu[s + 1]))
        if sl.stop == sl.start:
            continue
        one = oracle.varlen_bwd(q[sl], k[sl], v[sl], do[sl],
                                np.array([0, sl.stop - sl.start], np.int32), 0.5)
        for a, b in zip(full, one):
            np.testing.assert_array_equal(a[sl], b)


# ------------------------------------------------- fused QKV input with rotary prologue
# Mage-Flow page, section on fusion opportunities in the DiT block: one W_qkv projection
# whose output is split into q, k, v by chunk(3, dim=-1), then RoPE, then attention.
# The rotary variant is the rotate-half pairing (i, i + d/2) with per-token angle tables.

def test_bf16_rounding_is_one_rounding_to_nearest_even():
    cases = {
        1.0 + 2.0 ** -8: 0x3F80,                     # tie, even neighbour below
        1.0 + 3 * 2.0 ** -8: 0x3F82,                 # tie, even neighbour above
        -(1.0 + 2.0 ** -8): 0xBF80,
        1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F81,        # just above the tie
        1.0 + 2.0 ** -8 + 2.0 ** -25: 0x3F81,        # fp32 first would make this a tie -> 0x3F80
        0.0: 0x0000,
        3.0: 0x4040,
        255.5: 0x4380,                               # 8 significant bits: 255.5 -> 256
    }
    got = oracle.round_bf16_bits(np.array(list(cases.keys())))
    assert [int(g) for g in got] == list(cases.values())
    # on fp32 inputs (one rounding either way) it agrees with the generator's own rounding
    x = np.random.default_rng(5).standard_normal(20000).astype(np.float32) * 37.0
    np.testing.assert_array_equal(oracle.round_bf16_bits(x.astype(np.float64)), W.bf16_bits(x))
    np.testing.assert_array_equal(oracle.widen_bf16(W.bf16_bits(x)),
                                  W.bf16_to_f64(W.bf16_bits(x)))


def test_rope_is_complex_rotation_of_half_pairs():
    rng = np.random.default_rng(11)
    T, H, d = 9, 3, 16
    x = rng.standard_normal((T, H, d))
    ang = rng.uniform(-10, 10, size=(T, d // 2))
    y = oracle.rope(x, np.cos(ang), np.sin(ang))
    z = torch.complex(torch.from_numpy(x[..., : d // 2]), torch.from_numpy(x[..., d // 2:]))
    zr = z * torch.polar(torch.ones(T, 1, d // 2, dtype=torch.float64),
                         torch.from_numpy(ang)[:, None, :])
    np.testing.assert_allclose(y[..., : d // 2], zr.real.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(y[..., d // 2:], zr.imag.numpy(), rtol=0, atol=1e-13)


def test_rope_special_angles_compose_and_keep_pair_norms():
    rng = np.random.default_rng(12)
    T, H, d = 5, 2, 8
    x = rng.standard_normal((T, H, d))
    one, zero = np.ones((T, d // 2)), np.zeros((T, d // 2))
    np.testing.assert_array_equal(oracle.rope(x, one, zero), x)          # angle 0
    quarter = oracle.rope(x, zero, one)                                  # angle pi/2
    np.testing.assert_array_equal(quarter[..., :4], -x[..., 4:])
    np.testing.assert_array_equal(quarter[..., 4:], x[..., :4])
    a, b = rng.uniform(-3, 3, (T, d // 2)), rng.uniform(-3, 3, (T, d // 2))
    two = oracle.rope(oracle.rope(x, np.cos(a), np.sin(a)), np.cos(b), np.sin(b))
    np.testing.assert_allclose(two, oracle.rope(x, np.cos(a + b), np.sin(a + b)), atol=1e-13)
    y = oracle.rope(x, np.cos(a), np.sin(a))
    np.testing.assert_allclose(y[..., :4] ** 2 + y[..., 4:] ** 2, x[..., :4] ** 2 + x[..., 4:] ** 2,
                               atol=1e-13)


def test_rope_scores_depend_only_on_relative_position():
    # 1-D positions p with angles p * w_j: q at m and k at n score like q at m+s, k at n+s
    rng = np.random.default_rng(13)
    d = 32
    w = 10000.0 ** (-np.arange(d // 2) / (d // 2))
    q, k = rng.standard_normal((1, 1, d)), rng.standard_normal((1, 1, d))

    def score(m, n):
        am, an = (m * w)[None], (n * w)[None]
        return float(np.sum(oracle.rope(q, np.cos(am), np.sin(am)) *
                            oracle.rope(k, np.cos(an), np.sin(an))))
    for m, n, s in [(0, 3, 7), (5, 1, 100), (12, 12, 33)]:
        assert abs(score(m, n) - score(m + s, n + s)) < 1e-10
    assert abs(score(0, 3) - score(0, 4)) > 1e-3


def test_fused_qkv_chunks_are_q_then_k_then_v():
    w = W.make([13, 0, 40, 7], heads=3, head_dim=64, seed=21)
    qkv = W.fuse_qkv(w.q, w.k, w.v)
    assert qkv.shape == (w.total_tokens, 3, 3, 64)
    o, l = oracle.qkv_rope_fwd(qkv, w.cu_seqlens, w.scale)
    o_ref, l_ref = oracle.varlen_fwd(w.q, w.k, w.v, w.cu_seqlens, w.scale)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(l, l_ref)
    o_swap, _ = oracle.varlen_fwd(w.q, w.v, w.k, w.cu_seqlens, w.scale)
    assert np.max(np.abs(o - o_swap)) > 0.1


def test_fused_qkv_rope_with_exact_quarter_turns():
    # angles of whole quarter turns rotate bf16 values exactly, so the expected attention
    # is the plain attention of q and k rotated by complex multiplication with i^n
    w = W.make([33, 1, 70], heads=2, head_dim=64, seed=22)
    T, d = w.total_tokens, 64
    turns = np.random.default_rng(23).integers(0, 4, size=(T, d // 2))
    cos = np.cos(turns * np.pi / 2).round()
    sin = np.sin(turns * np.pi / 2).round()
    o, l = oracle.qkv_rope_fwd(W.fuse_qkv(w.q, w.k, w.v), w.cu_seqlens, w.scale, cos, sin)

    def turn(bits):
        x = torch.from_numpy(W.bf16_to_f64(bits))
        z = torch.complex(x[..., : d // 2], x[..., d // 2:]) * \
            (torch.tensor(1j, dtype=torch.complex128) ** torch.from_numpy(turns)[:, None, :])
        return W.bf16_bits(torch.cat([z.real, z.imag], -1).numpy().astype(np.float32))
    o_ref, l_ref = oracle.varlen_fwd(turn(w.q), turn(w.k), w.v, w.cu_seqlens, w.scale)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(l, l_ref)
    o_plain, _ = oracle.varlen_fwd(w.q, w.k, w.v, w.cu_seqlens, w.scale)
    assert np.max(np.abs(o - o_plain)) > 0.1


def test_fused_qkv_rope_rounds_rotated_q_and_k_to_bf16():
    w = W.make([20, 9], heads=2, head_dim=64, seed=24)
    cos, sin = W.rope_tables_2d(w.lengths, 64)
    o, _ = oracle.qkv_rope_fwd(W.fuse_qkv(w.q, w.k, w.v), w.cu_seqlens, w.scale, cos, sin)
    qr = oracle.rope(W.bf16_to_f64(w.q), cos, sin)
    kr = oracle.rope(W.bf16_to_f64(w.k), cos, sin)
    o_exact, _ = oracle.varlen_fwd(qr, kr, W.bf16_to_f64(w.v), w.cu_seqlens, w.scale)
    diff = np.max(np.abs(o - o_exact))
    assert 0 < diff < 2e-2      # only the bf16 rounding of the rotated q and k separates them
    with pytest.raises(ValueError):
        oracle.qkv_rope_fwd(W.fuse_qkv(w.q, w.k, w.v), w.cu_seqlens, w.scale, cos, None)


# ------------------------------------------------------------- block-sparse tile lists
# SparseAttn article: section 3.1 (softmax restricted to a retained key set), section 04
# (block accounting: a block with one allowed pair is computed whole; the printed table),
# section 05 (sliding tiles: a query tile shares a set of key tiles).

def _frame_position_masks(ex):
    same_frame = ex.frame[:, None] == ex.frame[None, :]
    same_pos = ex.pixel[:, None] == ex.pixel[None, :]
    return same_frame, same_pos


def test_block_accounting_of_the_temporal_mask_matches_the_printed_counts():
    """Section 04: the same-position mask in frame-major order covers 64 active 4x4 blocks
    (1024 computed positions for 256 allowed pairs, utilisation 0.25); in token-major order
    16 blocks, 256 positions, utilisation 1."""
    ex = W.worked_example()
    _, same_pos = _frame_position_masks(ex)
    _, st = oracle.block_lists_from_mask(same_pos, 4, 4)
    assert (st["pairs"], st["active_blocks"], st["computed"]) == (256, 64, 1024)
    assert st["utilisation"] == 0.25
    perm = np.argsort(ex.pixel, kind="stable")
    _, st2 = oracle.block_lists_from_mask(same_pos[np.ix_(perm, perm)], 4, 4)
    assert (st2["pairs"], st2["active_blocks"], st2["computed"], st2["utilisation"]) == (256, 16, 256, 1.0)


@pytest.mark.parametrize("mask_name,block,prefixes", [
    ("frame", 16, ("spatial_head_same_frame", "temporal_head_same_frame")),
    ("position", 1, ("spatial_head_same_position", "temporal_head_same_position")),
])
def test_blocksparse_reproduces_the_printed_table(worked, mask_name, block, prefixes):
    """Section 04 table, through block lists instead of packs: the same-frame mask is the
    diagonal of 16-token blocks; the same-position mask, in frame-major order, needs
    1-token blocks (every query lists the 4 keys of its position)."""
    ex = W.worked_example()
    q = np.ascontiguousarray(ex.q.transpose(1, 0, 2))
    v = np.ascontiguousarray(np.repeat(ex.v[:, None, :], 2, 1))
    same_frame, same_pos = _frame_position_masks(ex)
    lists, _ = oracle.block_lists_from_mask(same_frame if mask_name == "frame" else same_pos,
                                            block, block)
    o, l = oracle.varlen_fwd_blocksparse(q, q, v, [0, 64], 1.0 / math.sqrt(20), [[lists]],
                                         block_q=block, block_k=block)
    full_o, full_l = worked["full"]
    for head, prefix in enumerate(prefixes):
        _check(worked["gold"], prefix + "_retained_mass", float(np.exp(l[head] - full_l[head]).mean()))
        _check(worked["gold"], prefix + "_mse",
               float(np.mean((o[:, head, :] - full_o[:, head, :]) ** 2)))


def _random_layout(rng, lengths, heads_layout, bq, bk, p=0.4):
    lay = []
    for _ in range(heads_layout):
        segs = []
        for L in lengths:
            nkb = -(-L // bk)
            segs.append([[int(J) for J in rng.permutation(nkb) if rng.random() < p]
                         for _ in range(-(-L // bq))])
        lay.append(segs)
    return lay


@pytest.mark.parametrize("seed", range(3))
def test_blocksparse_matches_dense_masked_softmax(seed):
    """Brute force: a dense T x T score matrix with -inf outside the allowed (same segment,
    listed block) pairs, softmax in numpy; rows with no allowed key are zero / -inf."""
    rng = np.random.default_rng(40 + seed)
    lengths = [int(x) for x in rng.integers(0, 90, size=4)]
    T, H, d, bq, bk = sum(lengths), 3, 8, 16, 8
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    lay = _random_layout(rng, lengths, H if seed % 2 else 1, bq, bk)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    o, l = oracle.varlen_fwd_blocksparse(q, k, v, cu, 0.4, lay, block_q=bq, block_k=bk)
    for h in range(H):
        allowed = np.zeros((T, T), dtype=bool)
        hl = lay[h if len(lay) == H else 0]
        for s, L in enumerate(lengths):
            a = int(cu[s])
            for i in range(L):
                for J in hl[s][i // bq]:
                    allowed[a + i, a + J * bk:a + min((J + 1) * bk, L)] = True
        sc = np.where(allowed, 0.4 * q[:, h] @ k[:, h].T, -np.inf)
        has = allowed.any(axis=1)
        m = np.where(has, sc.max(axis=1), 0.0)
        w = np.where(allowed, np.exp(sc - m[:, None]), 0.0)
        z = w.sum(axis=1)
        ref = np.where(has[:, None], (w @ v[:, h]) / np.where(has, z, 1.0)[:, None], 0.0)
        np.testing.assert_allclose(o[:, h], ref, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l[h][has], (m + np.log(np.where(has, z, 1.0)))[has], rtol=0,
                                   atol=1e-13)
        assert np.all(np.isneginf(l[h][~has]))


def test_blocksparse_with_every_block_listed_is_dense_attention():
    w = W.make([300, 1, 0, 517], 2, 64, seed=41)
    lay = [[[list(range(-(-L // 64))) for _ in range(-(-L // 256))] for L in w.lengths]]
    o, l = oracle.varlen_fwd_blocksparse(w.q, w.k, w.v, w.cu_seqlens, w.scale, lay)
    o_ref, l_ref = oracle.varlen_fwd(w.q, w.k, w.v, w.cu_seqlens, w.scale)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-12)


def test_blocksparse_list_order_out_of_range_and_empty_rows():
    rng = np.random.default_rng(42)
    w = W.make([700, 90], 2, 64, seed=43)
    lay = _random_layout(rng, w.lengths, 1, 256, 64, p=0.6)
    lay[0][0][1] = []                                    # query block with no keys
    o, l = oracle.varlen_fwd_blocksparse(w.q, w.k, w.v, w.cu_seqlens, w.scale, lay)
    assert np.all(o[256:512] == 0) and np.all(np.isneginf(l[:, 256:512]))
    shuffled = [[[list(rng.permutation(r)) + [-1, 99] for r in seg] for seg in lay[0]]]
    o2, l2 = oracle.varlen_fwd_blocksparse(w.q, w.k, w.v, w.cu_seqlens, w.scale, shuffled)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, l, rtol=0, atol=1e-13)
    rows = np.array([0, 255, 256, 699, 700, 789])
    o3, l3 = oracle.varlen_fwd_blocksparse(w.q, w.k, w.v, w.cu_seqlens, w.scale, lay, rows=rows)
    np.testing.assert_allclose(o3, o[rows], rtol=0, atol=1e-14)   # BLAS may block rows differently
    np.testing.assert_allclose(l3, l[:, rows], rtol=0, atol=1e-13)
    bad = [[[r + r[:1] for r in seg] for seg in lay[0]]]
    with pytest.raises(ValueError):
        oracle.varlen_fwd_blocksparse(w.q, w.k, w.v, w.cu_seqlens, w.scale, bad)


# ---------------------------------------------------------------- FP8 P.V variant
# FPS Attention slides (tool.lu deck on accelerating multimodal generation, slides 35-38):
# V per channel, P per tensor, FP8 attention with dequantisation.  Readings: OCP e4m3,
# power-of-two V scales per (segment, head, channel), P scaled by 2^8.

def test_e4m3_rounding_matches_torch_float8():
    """torch's float8_e4m3fn conversion (round to nearest even) is an independent routine."""
    rng = np.random.default_rng(50)
    x = np.concatenate([rng.uniform(-448, 448, 4000), rng.uniform(-2.0 ** -5, 2.0 ** -5, 4000),
                        np.ldexp(rng.integers(-600, 600, 2000) + 0.5, -10),   # exact ties
                        np.ldexp(rng.integers(1, 64, 500) * 2 + 1, rng.integers(-4, 3, 500)),
                        [0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10]])
    x = x[np.abs(x) <= 448]
    x = x.astype(np.float32).astype(np.float64)          # torch converts from float32
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(oracle.e4m3_encode(oracle.e4m3_round(x)), ref.view(torch.uint8).numpy())
    np.testing.assert_array_equal(oracle.e4m3_round(x), ref.to(torch.float64).numpy())


def test_e4m3_codes_round_trip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    assert vals.max() == 448.0 and vals[codes == 0x01][0] == 2.0 ** -9
    back = oracle.e4m3_encode(vals)
    same = (back == codes) | ((codes == 0x80) & (back == 0x80))
    assert np.all(same)
    np.testing.assert_array_equal(oracle.e4m3_round(vals), vals)


def test_v_scale_exponent_is_the_smallest_that_fits():
    rng = np.random.default_rng(51)
    amax = np.concatenate([np.exp(rng.uniform(-20, 20, 5000)), [448.0, 449.0, 224.0, 1.0, 0.875 * 2 ** 9]])
    # (none of these is small enough for the -126 floor)
    e = oracle.v_scale_exponent(amax)
    assert np.all(amax * 2.0 ** -e <= 448.0) and np.all(amax * 2.0 ** -(e - 1) > 448.0)
    assert list(oracle.v_scale_exponent(np.array([448.0, 449.0, 0.0]))) == [0, 1, 0]
    assert list(oracle.v_scale_exponent(np.array([2.0 ** -120, 2.0 ** -133]))) == [-126, -126]


def test_quantize_v_per_segment_channel():
    w = W.make([40, 0, 33, 1], 3, 16, seed=52)
    v = W.bf16_to_f64(w.v)
    v[0:40, 1, 5] = 0.0                                   # an all-zero channel of segment 0
    vb = W.bf16_bits(v.astype(np.float32))
    codes, scales = oracle.quantize_v_fp8(vb, w.cu_seqlens)
    assert scales[0, 1, 5] == 1.0 and np.all(codes[0:40, 1, 5] == 0)
    deq = oracle.dequantize_v_fp8(codes, scales, w.cu_seqlens)
    vv = W.bf16_to_f64(vb)
    seg = np.searchsorted(w.cu_seqlens[1:], np.arange(w.total_tokens), side="right")
    step = np.maximum(np.abs(vv) * 2.0 ** -4, 2.0 ** -10 * scales[seg])
    assert np.all(np.abs(deq - vv) <= step + 1e-300)
    for s, (a, b) in enumerate(zip(w.cu_seqlens[:-1], w.cu_seqlens[1:])):   # segments alone
        if b > a:
            c1, s1 = oracle.quantize_v_fp8(vb[a:b], [0, b - a])
            np.testing.assert_array_equal(c1, codes[a:b])
            np.testing.assert_array_equal(s1[0], scales[s])
    m = np.abs(vv[40:73]).max(axis=0) / scales[2]          # the scale uses the fp8 range
    assert np.all((m > 224) & (m <= 448))


def test_fp8pv_blocked_steps_without_rounding_are_exact_attention():
    w = W.make([130, 1, 64, 200], 2, 32, seed=53)
    codes, scales = oracle.quantize_v_fp8(w.v, w.cu_seqlens)
    o, l = oracle.varlen_fwd_fp8pv_blocked(w.q, w.k, codes, scales, w.cu_seqlens, w.scale, quantize=False)
    vd = oracle.dequantize_v_fp8(codes, scales, w.cu_seqlens)
    o_ref, l_ref = oracle.varlen_fwd(W.bf16_to_f64(w.q), W.bf16_to_f64(w.k), vd, w.cu_seqlens, w.scale)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("qk_scale", [1.0, 4.0])
def test_fp8pv_blocked_steps_stay_within_the_bound(qk_scale):
    """The FP8 steps differ from exact attention on the dequantised V by at most the
    rounding of each weight (relative 2^-4, absolute 2^-10 in the 2^8-scaled units); the
    bound is reached to within a small factor, so it is not vacuous."""
    w = W.make([300, 77, 520], 2, 64, seed=54)
    q = W.bf16_bits((W.bf16_to_f64(w.q) * qk_scale).astype(np.float32))
    codes, scales = oracle.quantize_v_fp8(w.v, w.cu_seqlens)
    o, l = oracle.varlen_fwd_fp8pv_blocked(q, w.k, codes, scales, w.cu_seqlens, w.scale)
    vd = oracle.dequantize_v_fp8(codes, scales, w.cu_seqlens)
    o_ref, l_ref = oracle.varlen_fwd(W.bf16_to_f64(q), W.bf16_to_f64(w.k), vd, w.cu_seqlens, w.scale)
    bound = oracle.fp8pv_error_bound(q, w.k, codes, scales, w.cu_seqlens, w.scale)
    err = np.abs(o - o_ref)
    assert np.all(err <= bound * (1 + 1e-9) + 1e-13)
    assert (err / bound).max() > 0.1
    np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-12)     # LSE uses unrounded weights
    rows = np.array([0, 299, 300, 376, 377, 896])
    o2, l2 = oracle.varlen_fwd_fp8pv_blocked(q, w.k, codes, scales, w.cu_seqlens, w.scale, rows=rows)
    np.testing.assert_allclose(o2, o[rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(oracle.fp8pv_error_bound(q, w.k, codes, scales, w.cu_seqlens, w.scale,
                                                        rows=rows), bound[rows], rtol=1e-12, atol=0)


def test_fps_blocked_fp8_steps_over_block_lists():
    """FPS Attention = sliding-tile block lists + FP8 P.V (tool.lu deck, slides 35-38): the
    blocked FP8 steps visit only the listed key blocks.  Every block listed gives the dense
    steps; unrounded weights give exact block-sparse attention on the dequantised V; with
    rounding the result stays within the bound over the retained keys; an empty list gives
    a zero row and LSE = -inf."""
    rng = np.random.default_rng(55)
    w = W.make([700, 90, 300], 2, 64, seed=56)
    codes, scales = oracle.quantize_v_fp8(w.v, w.cu_seqlens)
    full = [[[list(range(-(-L // 64))) for _ in range(-(-L // 256))] for L in w.lengths]]
    o_d, l_d = oracle.varlen_fwd_fp8pv_blocked(w.q, w.k, codes, scales, w.cu_seqlens, w.scale)
    o_f, l_f = oracle.varlen_fwd_fp8pv_blocked(w.q, w.k, codes, scales, w.cu_seqlens, w.scale, layout=full)
    np.testing.assert_allclose(o_f, o_d, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l_f, l_d, rtol=0, atol=1e-13)
    lay = W.random_layout(rng, w.lengths, 2, density=0.5)
    lay[1][0][1] = []                                               # head 1, rows 256..511: no keys
    vd = oracle.dequantize_v_fp8(codes, scales, w.cu_seqlens)
    o_x, l_x = oracle.varlen_fwd_blocksparse(W.bf16_to_f64(w.q), W.bf16_to_f64(w.k), vd, w.cu_seqlens,
                                             w.scale, lay)
    o_u, l_u = oracle.varlen_fwd_fp8pv_blocked(w.q, w.k, codes, scales, w.cu_seqlens, w.scale,
                                               quantize=False, layout=lay)
    np.testing.assert_allclose(o_u, o_x, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_u[np.isfinite(l_x)], l_x[np.isfinite(l_x)], rtol=0, atol=1e-12)
    assert np.all(np.isneginf(l_u[1, 256:512])) and np.all(o_u[256:512, 1] == 0)
    o_q, l_q = oracle.varlen_fwd_fp8pv_blocked(w.q, w.k, codes, scales, w.cu_seqlens, w.scale, layout=lay)
    bound = oracle.fp8pv_error_bound(w.q, w.k, codes, scales, w.cu_seqlens, w.scale, layout=lay)
    err = np.abs(o_q - o_x)
    assert np.all(err <= bound * (1 + 1e-9) + 1e-13) and (err / np.maximum(bound, 1e-300)).max() > 0.1
