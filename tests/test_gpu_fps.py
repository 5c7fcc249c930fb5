"""GPU parity of FPS Attention (pfa_varlen_fwd_blocksparse_fp8pv): block-sparse key-block
lists with the P.V product in FP8, against exact block-sparse attention on the dequantised
V (within the FP8 bound over the retained keys) and the oracle's blocked FP8 steps over the
same lists, through the C ABI."""
import numpy as np
import pytest

import oracle
import pfa_workloads as W
from tests._gpu import KERNEL_ALLOWANCE, LSE_ABS, bf16_half_ulp, from_dev_bf16, say, to_dev
from tests.test_gpu_fp8 import EMUL_REL_RMS

pytestmark = pytest.mark.gpu


def _run(wl, layout, label, rows=None):
    import torch
    from packed_varlen_flash_amd import (block_layout_csr, pfa_quantize_v_fp8,
                                         pfa_varlen_fwd_blocksparse_fp8pv)
    kv_ptr, kv_idx, lh = block_layout_csr(layout, wl.lengths, wl.max_seqlen)
    say(f"[gpu] pfa_varlen_fwd_blocksparse_fp8pv {label}: segs={wl.num_seqs} T={wl.total_tokens} "
        f"H={wl.heads} d={wl.head_dim} layout_heads={lh} nnz={kv_idx.shape[0]}")
    cu = torch.from_numpy(wl.cu_seqlens).to("cuda")
    v8, vs = pfa_quantize_v_fp8(to_dev(wl.v), cu)
    out, lse = pfa_varlen_fwd_blocksparse_fp8pv(to_dev(wl.q), to_dev(wl.k), v8, vs, cu, wl.max_seqlen,
                                                torch.from_numpy(kv_ptr).to("cuda"),
                                                torch.from_numpy(kv_idx).to("cuda"), lh, wl.scale)
    torch.cuda.synchronize()
    o = W.bf16_to_f64(from_dev_bf16(out))
    lse = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        o, lse = o[rows], lse[:, rows]
    return o, lse


def _check(wl, layout, label, rows=None):
    o, lse = _run(wl, layout, label, rows)
    codes, scales = oracle.quantize_v_fp8(wl.v, wl.cu_seqlens)
    vd = oracle.dequantize_v_fp8(codes, scales, wl.cu_seqlens)
    o_ex, l_ex = oracle.varlen_fwd_blocksparse(W.bf16_to_f64(wl.q), W.bf16_to_f64(wl.k), vd,
                                               wl.cu_seqlens, wl.scale, layout, rows=rows)
    bound = oracle.fp8pv_error_bound(wl.q, wl.k, codes, scales, wl.cu_seqlens, wl.scale, rows=rows,
                                     layout=layout)
    empty = np.isneginf(l_ex)
    assert np.all(o[empty.T] == 0.0) and np.all(np.isneginf(lse[empty]))
    err = np.abs(o - o_ex)
    allow = bound + bf16_half_ulp(np.abs(o_ex) + bound) + KERNEL_ALLOWANCE
    worst = float((err - allow).max())
    lse_err = float(np.abs(np.where(empty, 0.0, lse) - np.where(empty, 0.0, l_ex)).max())
    o_em, _ = oracle.varlen_fwd_fp8pv_blocked(wl.q, wl.k, codes, scales, wl.cu_seqlens, wl.scale,
                                              rows=rows, layout=layout)
    rr = float(np.sqrt(((o - o_em) ** 2).sum() / (o_em ** 2).sum()))
    say(f"[parity] {label}: max|err| vs exact {err.max():.3e}, worst excess {worst:.3e}, "
        f"LSE {lse_err:.3e}, relRMS vs the FP8 steps {rr:.3e}")
    assert worst <= 0.0
    assert lse_err <= LSE_ABS
    assert rr <= EMUL_REL_RMS


@pytest.mark.parametrize("seed", range(4))
def test_random_layouts_full(seed):
    rng = np.random.default_rng(500 + seed)
    lengths = W.random_lengths(rng, int(rng.integers(1, 6)), 1400)
    if sum(lengths) == 0:
        lengths[0] = 1
    wl = W.make(lengths, 3, 64 if seed % 2 else 128, seed=500 + seed)
    lay = W.random_layout(rng, wl.lengths, wl.heads if seed % 2 == 0 else 1, density=0.5)
    lay[0][0] = [row + [-1, 4000] for row in lay[0][0]]        # out-of-range entries are skipped
    _check(wl, lay, f"random layout seed={seed} L={wl.lengths}")


def test_c3_band_sampled():
    wl = W.generate("C3")
    lay = W.band_layout(wl.lengths, radius=1024)
    rows = W.sample_rows(wl.cu_seqlens, stride=61, edge=64, full_upto=0)
    _check(wl, lay, f"C3 band +-1024, FP8, sampled {len(rows)} rows", rows=rows)


def test_every_block_listed_equals_the_dense_fp8_kernel_bitwise():
    import torch
    from packed_varlen_flash_amd import pfa_quantize_v_fp8, pfa_varlen_fwd_fp8pv
    wl = W.make([1024, 300, 1, 0, 700], 2, 128, seed=510)
    full = [[[list(range(-(-L // 64))) for _ in range(-(-L // 256))] for L in wl.lengths]]
    o, lse = _run(wl, full, "every block listed")
    cu = torch.from_numpy(wl.cu_seqlens).to("cuda")
    v8, vs = pfa_quantize_v_fp8(to_dev(wl.v), cu)
    out2, lse2 = pfa_varlen_fwd_fp8pv(to_dev(wl.q), to_dev(wl.k), v8, vs, cu, wl.max_seqlen, wl.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o, W.bf16_to_f64(from_dev_bf16(out2)))
    np.testing.assert_array_equal(lse, lse2.cpu().numpy().astype(np.float64))


def test_empty_rows():
    wl = W.make([500, 37], 2, 128, seed=511)
    _check(wl, [[[[0, 1], []], [[0]]]], "one empty query block")
