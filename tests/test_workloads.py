"""The seeded generator: sizes of the named workloads, determinism, row samples."""
import hashlib

import numpy as np

import pfa_workloads as W


def test_config_sizes():
    T = {n: sum(c.lengths) for n, c in W.CONFIGS.items()}
    assert T == {"C1": 320, "C2": 32768, "C3": 39248, "C4": 32768, "C5a": 65536, "C5b": 87313}
    c3 = W.CONFIGS["C3"]
    assert sorted(c3.lengths) == sorted([4096] * 7 + [1296] * 5 + [1024] * 4)
    assert W.flops(c3.lengths, 24, 128) == 4 * sum(L * L for L in c3.lengths) * 24 * 128


def test_generation_is_deterministic():
    a = W.generate("C1")
    b = W.generate("C1")
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        assert hashlib.sha256(x.tobytes()).digest() == hashlib.sha256(y.tobytes()).digest()
    c = W.generate("C1", seed=1)
    assert not np.array_equal(a.q, c.q)
    assert a.q.dtype == np.uint16 and a.q.shape == (320, 4, 64)
    assert list(a.cu_seqlens) == [0, 256, 320]


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38], np.float32)
    bits = W.bf16_bits(x)
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x7F62]
    assert np.all(W.bf16_to_f32(bits)[[0, 3]] == x[[0, 3]])


def test_sharp_heads_scale_q_and_k():
    wl = W.make([64], 24, 128, seed=0, per_head_qk_scale=True)
    plain = W.make([64], 24, 128, seed=0)
    q0, q23 = W.bf16_to_f32(wl.q[:, 0]), W.bf16_to_f32(wl.q[:, 23])
    p0, p23 = W.bf16_to_f32(plain.q[:, 0]), W.bf16_to_f32(plain.q[:, 23])
    assert np.allclose(q0, 0.5 * p0, rtol=1e-2, atol=1e-2)
    assert np.allclose(q23, 2.0 * p23, rtol=1e-2, atol=1e-2)
    assert np.array_equal(wl.v, plain.v)


def test_row_sample():
    cu = W.cu_from_lengths([5000, 100])
    rows = W.sample_rows(cu, stride=61, edge=64, full_upto=200)
    assert rows[0] == 0 and 4999 in rows and 63 in rows and 64 not in rows and 61 in rows
    assert np.all(np.isin(np.arange(5000, 5100), rows))
    assert np.all(np.diff(rows) > 0)


def test_grid_positions_and_rope_tables():
    r, c = W.grid_positions([4096, 1296, 5])
    assert (r[4095], c[4095]) == (63, 63) and (r[4096 + 1295], c[4096 + 1295]) == (35, 35)
    assert list(r[-5:]) == [0, 0, 0, 1, 1] and list(c[-5:]) == [0, 1, 2, 0, 1]
    cos, sin = W.rope_tables_2d([4096, 5], 128)
    assert cos.shape == (4101, 64) and cos.dtype == np.float32
    assert np.all(cos[0] == 1) and np.all(sin[0] == 0) and np.all(cos[4096] == 1)
    np.testing.assert_allclose(cos ** 2 + sin ** 2, 1, atol=1e-6)
    assert sin[70, 0] == np.float32(np.sin(1.0)) and sin[70, 32] == np.float32(np.sin(6.0))


def test_band_layout_and_pair_count():
    lay = W.band_layout([4096, 100, 0], radius=1024)
    rows = lay[0][0]
    assert len(rows) == 16 and rows[0] == list(range(0, 20)) and rows[8] == list(range(16, 52))
    assert rows[15] == list(range(44, 64))
    assert lay[0][1] == [[0, 1]] and lay[0][2] == []
    full = [[[list(range(64))] * 16]]
    assert W.layout_pairs(full, [4096], heads=3) == 3 * 4096 * 4096
    assert W.layout_pairs(lay, [4096, 100, 0], heads=1) == \
        sum(256 * 64 * len(r) for r in rows) + 100 * 100
