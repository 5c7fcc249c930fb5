"""HIP path vs the fp64 oracle, through the C ABI, on seeded inputs.

Bars (bf16 inputs): output max |err| <= 1e-2 and relative RMS <= 4e-3, LSE max |err|
<= 1e-3, element by element.  Small cases are compared in full; the full-size workloads
run in the same launch configuration the benchmark times and are compared on a
deterministic row sample the oracle computes one row at a time.
"""
import math

import numpy as np
import pytest

import oracle
import pfa_workloads as W
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _full_check(wl, label):
    out, lse = G.run(wl, label)
    o_ref, l_ref = oracle.varlen_fwd(wl.q, wl.k, wl.v, wl.cu_seqlens, wl.scale)
    G.assert_parity(G.compare(out, lse, o_ref, l_ref), label)
    return out, lse


def test_c1_two_images_full():
    wl = W.generate("C1")
    _full_check(wl, "C1 [256,64] H4 d64")


@pytest.mark.parametrize("seed", range(10))
def test_random_ragged_packs_full(seed):
    rng = np.random.default_rng(1000 + seed)
    d = [64, 128][seed % 2]
    H = [1, 3, 2, 5][seed % 4]
    lengths = W.random_lengths(rng, int(rng.integers(1, 9)), [70, 300, 700, 1300][seed % 4])
    if sum(lengths) == 0:
        lengths.append(5)
    wl = W.make(lengths, H, d, seed=seed, name=f"ragged{seed}",
                scale=[None, 0.05, 0.3][seed % 3])
    _full_check(wl, f"ragged seed={seed} d={d} H={H} lens={lengths}")


@pytest.mark.parametrize("lengths", [[1], [64], [65], [255, 256, 257], [511, 512, 513], [1, 1, 1, 2]])
def test_tile_boundaries_full(lengths):
    for d in (64, 128):
        wl = W.make(lengths, 2, d, seed=7, name=f"edges{lengths}")
        _full_check(wl, f"edges {lengths} d={d}")


def test_many_segments_bitonic_schedule():
    """Over 512 segments the schedule is sorted by a bitonic network in LDS (capacity 2048
    here)."""
    rng = np.random.default_rng(5)
    lengths = [int(x) for x in rng.integers(0, 40, size=1100)]
    wl = W.make(lengths, 2, 64, seed=5, name="1100 segments")
    _full_check(wl, "1100 segments d64")


@pytest.mark.parametrize("n,d", [(4096, 128), (4097, 64), (5000, 128)])
def test_segments_at_and_beyond_the_sort_capacity(n, d):
    """4,096 segments fill the largest schedule capacity; above it the kernel walks the
    unsorted (segment, head, tile) slots."""
    rng = np.random.default_rng(8 + n)
    lengths = [int(x) for x in rng.integers(0, 48, size=n)]
    lengths[int(rng.integers(0, n))] = 700          # one multi-tile segment among them
    wl = W.make(lengths, 1, d, seed=8 + n, name=f"{n} segments")
    _full_check(wl, f"{n} segments d{d}")


def test_many_segments_sorted_mode():
    rng = np.random.default_rng(6)
    lengths = [int(x) for x in rng.integers(0, 300, size=1000)]
    wl = W.make(lengths, 1, 128, seed=6, name="1000 segments")
    _full_check(wl, "1000 segments d128")


SAMPLED = {
    # config: (stride, edge, full_upto) of the row sample
    "C2": (61, 64, 0),
    "C3": (61, 64, 0),
    "C4": (61, 64, 0),
    "C5a": (509, 64, 0),
    "C5b": (509, 64, 1296),
}


@pytest.mark.parametrize("name", list(SAMPLED))
def test_full_size_workloads_sampled(name):
    wl = W.generate(name)
    out, lse = G.run(wl, name)
    stride, edge, full_upto = SAMPLED[name]
    rows = W.sample_rows(wl.cu_seqlens, stride=stride, edge=edge, full_upto=full_upto)
    G.say(f"[oracle] {name}: {len(rows)} sampled rows")
    o_ref, l_ref = oracle.varlen_fwd(wl.q, wl.k, wl.v, wl.cu_seqlens, wl.scale, rows=rows)
    G.assert_parity(G.compare(out[rows], lse[:, rows], o_ref, l_ref), f"{name} sampled")


def test_single_token_segment_returns_value_exactly():
    wl = W.make([1, 37, 1, 129], 3, 128, seed=11, name="L=1")
    out, lse = G.run(wl)
    for t in (0, 38):
        assert np.array_equal(out[t], wl.v[t])
        qf, kf = W.bf16_to_f64(wl.q[t]), W.bf16_to_f64(wl.k[t])
        np.testing.assert_allclose(lse[:, t], wl.scale * np.sum(qf * kf, axis=1), atol=1e-4)


def test_pack_equals_each_segment_alone_bitwise():
    lengths = [300, 77, 1, 0, 513, 64]
    for d in (64, 128):
        wl = W.make(lengths, 2, d, seed=21, name="pack")
        out, lse = G.run(wl, f"pack d={d}")
        cu = wl.cu_seqlens
        for s, L in enumerate(lengths):
            if L == 0:
                continue
            a, b = int(cu[s]), int(cu[s + 1])
            one = W.Workload(name="alone", q=wl.q[a:b], k=wl.k[a:b], v=wl.v[a:b],
                             cu_seqlens=np.array([0, L], np.int32), lengths=(L,), heads=2,
                             head_dim=d, scale=wl.scale, max_seqlen=L, seed=21)
            o1, l1 = G.run(one, f"segment {s} alone d={d}")
            assert np.array_equal(out[a:b], o1) and np.array_equal(lse[:, a:b], l1)


@pytest.mark.parametrize("poison", [np.nan, np.inf, 1e30])
def test_poisoned_neighbours_do_not_leak(poison):
    lengths = [200, 333, 129]
    wl = W.make(lengths, 2, 128, seed=31, name="poison")
    out, lse = G.run(wl, "clean")
    a, b = int(wl.cu_seqlens[1]), int(wl.cu_seqlens[2])
    pb = W.bf16_bits(np.array([poison], dtype=np.float32))[0] if np.isfinite(poison) else \
        np.array([poison], dtype=np.float32).view(np.uint32)[0] >> 16
    q, k, v = wl.q.copy(), wl.k.copy(), wl.v.copy()
    for arr in (q, k, v):
        arr[:a] = pb
        arr[b:] = pb
    wl2 = W.Workload(name="poisoned", q=q, k=k, v=v, cu_seqlens=wl.cu_seqlens, lengths=wl.lengths,
                     heads=2, head_dim=128, scale=wl.scale, max_seqlen=wl.max_seqlen, seed=31)
    out2, lse2 = G.run(wl2, f"poisoned with {poison}")
    assert np.array_equal(out2[a:b], out[a:b]) and np.array_equal(lse2[:, a:b], lse[:, a:b])


def test_run_to_run_bitwise_determinism():
    wl = W.generate("C1")
    dev = G.upload(wl)
    o1, l1 = G.run(wl, "C1 run 1", dev=dev)
    o2, l2 = G.run(wl, "C1 run 2", dev=dev)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_lse_is_optional():
    wl = W.make([100, 50], 2, 64, seed=41)
    dev = G.upload(wl)
    o1, l1 = G.run(wl, "with lse", dev=dev)
    o2, l2 = G.run(wl, "without lse", dev=dev, want_lse=False)
    assert l2 is None and np.array_equal(o1, o2)


def test_guard_regions_untouched():
    """Outputs are written only inside [0, T) rows: sentinels around out and lse survive."""
    import ctypes
    import torch
    from packed_varlen_flash_amd import _lib
    wl = W.make([130, 1, 66], 3, 128, seed=51)
    q, k, v, cu = G.upload(wl)
    T, H, d = wl.total_tokens, wl.heads, wl.head_dim
    guard = 4096
    out_buf = torch.full((guard + T * H * d + guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_buf = torch.full((guard + H * T + guard,), -12345.0, dtype=torch.float32, device="cuda")
    G.say("[gpu] pfa_varlen_fwd guard-region case")
    rc = _lib.load().pfa_varlen_fwd(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        ctypes.c_void_p(cu.data_ptr()), 3, wl.max_seqlen, H, d, wl.scale,
        ctypes.c_void_p(out_buf.data_ptr() + 2 * guard), ctypes.c_void_p(lse_buf.data_ptr() + 4 * guard),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    ob = out_buf.float().cpu().numpy()
    lb = lse_buf.cpu().numpy()
    assert np.all(np.isnan(ob[:guard])) and np.all(np.isnan(ob[guard + T * H * d:]))
    assert not np.any(np.isnan(ob[guard:guard + T * H * d]))
    assert np.all(lb[:guard] == -12345.0) and np.all(lb[guard + H * T:] == -12345.0)
    o_ref, l_ref = oracle.varlen_fwd(wl.q, wl.k, wl.v, wl.cu_seqlens, wl.scale)
    body = out_buf[guard:guard + T * H * d].view(torch.int16).cpu().numpy().view(np.uint16).reshape(T, H, d)
    G.assert_parity(G.compare(body, lb[guard:guard + H * T].reshape(H, T), o_ref, l_ref), "guard body")


def test_side_stream():
    import torch
    wl = W.make([257, 100], 2, 128, seed=61)
    s = torch.cuda.Stream()
    dev = G.upload(wl)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out, lse = G.run(wl, "side stream", dev=dev, stream=s)
    o_ref, l_ref = oracle.varlen_fwd(wl.q, wl.k, wl.v, wl.cu_seqlens, wl.scale)
    G.assert_parity(G.compare(out, lse, o_ref, l_ref), "side stream")


def test_sharp_softmax_heads():
    """C4's per-head Q/K scaling at a small size: logits with std up to 4."""
    wl = W.make([1024, 700], 24, 128, seed=71, per_head_qk_scale=True, name="sharp")
    _full_check(wl, "sharp heads [1024,700] H24")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", [1.0, 3.0])
def test_running_max_jumps_inside_a_stage(d, scale):
    """Large scales make the running max jump by more than 2^8 in many sub-blocks (both
    halves of a 64-key stage), exercising every rescale path of the online softmax."""
    wl = W.make([37, 100, 300, 64, 129], 3, d, seed=81, scale=scale, name="max jumps")
    _full_check(wl, f"max jumps d={d} scale={scale}")


def test_tensors_beyond_two_giga_elements():
    """q, k, v and out of 2.26e9 elements each (above the 32-bit element index range):
    538 segments of 4096 tokens, 8 heads, d 128, built from three seeded segment blocks
    (segment s holds block s mod 3, so an index that wrapped at 2^31 elements would land
    on a segment of another block).  Checked against the oracle on sampled rows of the
    segments just below and above the 2^31-element boundary and of the last segment, and
    every sampled segment bitwise against the same block's first segment."""
    import torch
    from packed_varlen_flash_amd import pfa_varlen_fwd
    L, H, d, n = 4096, 8, 128, 538
    T = L * n
    assert T * H * d > 2 ** 31
    blocks = [W.make([L], H, d, seed=900 + c, name=f"block{c}") for c in range(3)]
    idx = torch.arange(n, device="cuda") % 3
    big = []
    for name in ("q", "k", "v"):
        stack = torch.stack([G.to_dev(getattr(b, name)) for b in blocks])
        big.append(stack[idx].reshape(T, H, d))
        del stack
    cu = torch.arange(0, T + 1, L, dtype=torch.int32, device="cuda")
    G.say(f"[gpu] pfa_varlen_fwd beyond 2^31 elements: segs={n} T={T} H={H} d={d}")
    out, lse = pfa_varlen_fwd(big[0], big[1], big[2], cu, L, blocks[0].scale)
    torch.cuda.synchronize()
    rows = W.sample_rows(blocks[0].cu_seqlens, stride=97, edge=16, full_upto=0)
    refs = {}
    for c, b in enumerate(blocks):
        refs[c] = oracle.varlen_fwd(b.q, b.k, b.v, b.cu_seqlens, b.scale, rows=rows)
    first = {c: G.from_dev_bf16(out[c * L:(c + 1) * L]) for c in range(3)}
    for s in (511, 512, 537):          # 512 * 4096 * 8 * 128 = 2^31 elements
        c = s % 3
        ob = G.from_dev_bf16(out[s * L:(s + 1) * L])
        ls = lse[:, s * L:(s + 1) * L].cpu().numpy()
        np.testing.assert_array_equal(ob, first[c])
        o_ref, l_ref = refs[c]
        G.assert_parity(G.compare(ob[rows], ls[:, rows], o_ref, l_ref), f"segment {s} (block {c})")
    del big, out, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("d,bound", [(128, 256), (64, 128)])
def test_short_segments_resident_kernel_equals_streaming(d, bound):
    """max_seqlen only selects the kernel: at most the resident bound (256 keys at d = 128,
    128 at d = 64) each segment's K/V are loaded into LDS whole, one above it they stream in
    64-key stages.  Both must give the same bits, and match the oracle."""
    import dataclasses
    rng = np.random.default_rng(90 + d)
    lengths = rng.integers(0, bound + 1, size=300).tolist()
    lengths[:4] = [bound, 1, 0, bound - 1]
    wl = W.make(lengths, 3, d, seed=90 + d, name="short")
    assert wl.max_seqlen <= bound
    dev = G.upload(wl)
    o_res, l_res = G.run(wl, f"resident (max_seqlen {wl.max_seqlen}) d={d}", dev=dev)
    o_str, l_str = G.run(dataclasses.replace(wl, max_seqlen=bound + 1), f"streaming (max_seqlen {bound + 1}) d={d}", dev=dev)
    assert np.array_equal(o_res, o_str) and np.array_equal(l_res.view(np.uint32), l_str.view(np.uint32))
    o_ref, l_ref = oracle.varlen_fwd(wl.q, wl.k, wl.v, wl.cu_seqlens, wl.scale)
    G.assert_parity(G.compare(o_res, l_res, o_ref, l_ref), f"short segments d={d}")


def test_d64_four_and_eight_wave_tiles_agree_bitwise():
    """At d = 64 a query bound of 512 rows or more selects 512-query tiles of eight waves,
    below it 256-query tiles of four.  max_seqlen is only a bound, so the same pack (every
    segment under 512 rows) run with 511 and with 512 must give the same bits, for the
    self-attention, separate-table and fused-QKV entry points."""
    import torch
    from packed_varlen_flash_amd import pfa_varlen_fwd, pfa_varlen_fwd_qk, pfa_varlen_fwd_qkv
    rng = np.random.default_rng(95)
    lengths = rng.integers(0, 512, size=40).tolist()
    lengths[:3] = [511, 257, 1]
    wl = W.make(lengths, 3, 64, seed=95, name="d64 tiles")
    q, k, v, cu = G.upload(wl)
    cu_k = cu.clone()       # a second table: the cross mode (a key bound of 511 or 512 is
                            # above the resident kernel's 128 keys, so it streams K/V)
    qkv = torch.stack([q, k, v], dim=1).contiguous()   # [T, 3, H, d]
    res = {}
    for bound in (511, 512):
        o1, l1 = pfa_varlen_fwd(q, k, v, cu, bound, wl.scale)
        o2, l2 = pfa_varlen_fwd_qk(q, k, v, cu, cu_k, bound, bound, wl.scale)
        o3, l3, _ = pfa_varlen_fwd_qkv(qkv, cu, bound, wl.scale)
        torch.cuda.synchronize()
        res[bound] = [t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu()
                      for t in (o1, l1, o2, l2, o3, l3)]
        G.say(f"[gpu] d=64 self / cross / fused-QKV with max_seqlen {bound}")
    for a, b in zip(res[511], res[512]):
        assert torch.equal(a, b)
    assert torch.equal(res[511][0], res[511][2]) and torch.equal(res[511][0], res[511][4])
    o_ref, l_ref = oracle.varlen_fwd(wl.q, wl.k, wl.v, wl.cu_seqlens, wl.scale)
    out = res[512][0].numpy().view(np.uint16)
    G.assert_parity(G.compare(out, res[512][1].numpy().view(np.float32), o_ref, l_ref), "d=64 eight-wave tiles")
