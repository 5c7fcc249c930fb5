"""Packs that hold no tokens, and cross-attention whose key table holds no keys, through
every entry point and the C ABI: the kernels get no rows, outputs come back with their
(empty) shapes, and outputs that are not empty follow the conventions the oracle fixes
(a query without keys: O = 0 and LSE = -inf; an empty segment's V scale is 1)."""
import numpy as np
import pytest

import oracle
import pfa_workloads as W
from tests._gpu import from_dev_bf16, say, to_dev

pytestmark = pytest.mark.gpu


def _dev(arr):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr)).to("cuda")


@pytest.mark.parametrize("d", [64, 128])
def test_every_entry_point_on_a_pack_without_tokens(d):
    import torch
    import packed_varlen_flash_amd as P
    wl = W.make([0, 0, 0], 3, d, seed=7, name="no tokens")
    say(f"[gpu] empty pack d={d}: cu={wl.cu_seqlens.tolist()}")
    cu = _dev(wl.cu_seqlens)
    q, k, v = to_dev(wl.q), to_dev(wl.k), to_dev(wl.v)
    H = wl.heads

    out, lse = P.pfa_varlen_fwd(q, k, v, cu, 1)
    assert out.shape == (0, H, d) and lse.shape == (H, 0)
    out, lse = P.pfa_varlen_fwd_qk(q, k, v, cu, cu, 1, 1)
    assert out.shape == (0, H, d) and lse.shape == (H, 0)
    qkv = to_dev(W.fuse_qkv(wl.q, wl.k, wl.v))
    tab = torch.zeros((0, d // 2), dtype=torch.float32, device="cuda")
    for cos, sin in ((None, None), (tab, tab.clone())):
        out, lse, k_rot = P.pfa_varlen_fwd_qkv(qkv, cu, 1, rope_cos=cos, rope_sin=sin)
        assert out.shape == (0, H, d) and lse.shape == (H, 0)
        assert (k_rot is None) == (cos is None)
    kv_ptr, kv_idx, lh = P.block_layout_csr([[[] for _ in wl.lengths]], wl.lengths, 1)
    out, lse = P.pfa_varlen_fwd_blocksparse(q, k, v, cu, 1, _dev(kv_ptr), _dev(kv_idx), lh)
    assert out.shape == (0, H, d) and lse.shape == (H, 0)
    v8, vs = P.pfa_quantize_v_fp8(v, cu)
    out, lse = P.pfa_varlen_fwd_fp8pv(q, k, v8, vs, cu, 1)
    assert out.shape == (0, H, d) and lse.shape == (H, 0)
    out, lse = P.pfa_varlen_fwd_blocksparse_fp8pv(q, k, v8, vs, cu, 1, _dev(kv_ptr), _dev(kv_idx), lh)
    assert out.shape == (0, H, d) and lse.shape == (H, 0)
    o_m, l_m = P.pfa_attn_merge(out, lse, out, lse)
    assert o_m.shape == (0, H, d) and l_m.shape == (H, 0)
    dq, dk, dv = P.pfa_varlen_bwd(q, k, v, out, out, lse, cu, 1)
    assert dq.shape == dk.shape == dv.shape == (0, H, d)
    torch.cuda.synchronize()
    # the quantiser still writes every segment's scale: empty segments get 2^0
    codes, scales = oracle.quantize_v_fp8(wl.v, wl.cu_seqlens)
    assert v8.shape == codes.shape
    np.testing.assert_array_equal(vs.cpu().numpy().astype(np.float64), scales)


@pytest.mark.parametrize("d", [64, 128])
def test_cross_attention_with_no_keys_at_all(d):
    import torch
    from packed_varlen_flash_amd import pfa_varlen_fwd_qk
    wq = W.make([5, 300, 0, 7], 2, d, seed=8, name="queries")
    wk = W.make([0, 0, 0, 0], 2, d, seed=9, name="no keys")
    say(f"[gpu] cross without keys d={d}: Lq={wq.lengths}")
    out, lse = pfa_varlen_fwd_qk(to_dev(wq.q), to_dev(wk.k), to_dev(wk.v), _dev(wq.cu_seqlens),
                                 _dev(wk.cu_seqlens), wq.max_seqlen, 1)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.varlen_fwd_qk(wq.q, wk.k, wk.v, wq.cu_seqlens, wk.cu_seqlens, wq.scale)
    assert np.all(o_ref == 0.0) and np.all(np.isneginf(l_ref))
    assert np.all(W.bf16_to_f64(from_dev_bf16(out)) == 0.0)
    assert np.all(np.isneginf(lse.cpu().numpy()))
