"""The Python binding rejects caller-supplied buffers on the wrong device, of the wrong
dtype, shape or layout with ValueError before anything is launched (the library receives
only addresses, so such a buffer would otherwise be written out of bounds)."""
import numpy as np
import pytest

import pfa_workloads as W
from tests import _gpu as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def inputs():
    import torch
    wl = W.make([70, 30], 2, 64, seed=901)
    q, k, v, cu = G.upload(wl)
    return wl, q, k, v, cu, torch


def test_forward_rejects_host_and_misshaped_outputs(inputs):
    from packed_varlen_flash_amd import pfa_varlen_fwd, pfa_varlen_fwd_qk
    wl, q, k, v, cu, torch = inputs
    T, H, d = q.shape
    bad = {
        "out on the host": dict(out=torch.empty((T, H, d), dtype=torch.bfloat16)),
        "out fp32": dict(out=torch.empty((T, H, d), dtype=torch.float32, device="cuda")),
        "out short": dict(out=torch.empty((T - 1, H, d), dtype=torch.bfloat16, device="cuda")),
        "out strided": dict(out=torch.empty((T, H, 2 * d), dtype=torch.bfloat16, device="cuda")[:, :, :d]),
        "lse on the host": dict(lse=torch.empty((H, T), dtype=torch.float32)),
        "lse transposed": dict(lse=torch.empty((T, H), dtype=torch.float32, device="cuda")),
        "lse bf16": dict(lse=torch.empty((H, T), dtype=torch.bfloat16, device="cuda")),
    }
    for label, kw in bad.items():
        with pytest.raises(ValueError):
            pfa_varlen_fwd(q, k, v, cu, wl.max_seqlen, wl.scale, **kw)
        with pytest.raises(ValueError):
            pfa_varlen_fwd_qk(q, k, v, cu, cu, wl.max_seqlen, wl.max_seqlen, wl.scale, **kw)
    with pytest.raises(ValueError):
        pfa_varlen_fwd(q, k, v, cu.cpu(), wl.max_seqlen, wl.scale)    # table on the host


def test_merge_rejects_bad_lse_and_out(inputs):
    from packed_varlen_flash_amd import pfa_attn_merge, pfa_varlen_fwd
    wl, q, k, v, cu, torch = inputs
    o, l = pfa_varlen_fwd(q, k, v, cu, wl.max_seqlen, wl.scale)
    T, H, d = o.shape
    for lse in (torch.empty((H, T - 1), device="cuda"), torch.empty((H, T)),
                torch.empty((H, T), dtype=torch.float64, device="cuda")):
        with pytest.raises(ValueError):
            pfa_attn_merge(o, l, o, l, lse=lse)
    with pytest.raises(ValueError):
        pfa_attn_merge(o, l, o, l[:, : T - 1].contiguous())
    with pytest.raises(ValueError):
        pfa_attn_merge(o, l, o, l, out=torch.empty((T, H, d), dtype=torch.bfloat16))
    out, lse = pfa_attn_merge(o, l, o, l)          # the well-formed call still works
    torch.cuda.synchronize()
    assert out.shape == o.shape and lse.shape == l.shape


def test_backward_rejects_bad_buffers(inputs):
    from packed_varlen_flash_amd import pfa_varlen_bwd, pfa_varlen_fwd
    wl, q, k, v, cu, torch = inputs
    o, l = pfa_varlen_fwd(q, k, v, cu, wl.max_seqlen, wl.scale)
    dout = torch.ones_like(o)
    T, H, d = q.shape
    cases = [dict(lse=l.cpu()), dict(dq=torch.empty((T, H, d), dtype=torch.bfloat16)),
             dict(dv=torch.empty((T, H, d), dtype=torch.float32, device="cuda")),
             dict(workspace=torch.empty((2, H, T))),
             dict(workspace=torch.empty((2 * H * T + 5,), device="cuda")),
             dict(workspace=torch.empty((2, H, T), dtype=torch.float64, device="cuda"))]
    for kw in cases:
        args = dict(lse=l)
        args.update(kw)
        with pytest.raises(ValueError):
            pfa_varlen_bwd(q, k, v, o, dout, args.pop("lse"), cu, wl.max_seqlen, wl.scale, **args)


def test_offset_views_are_rejected_by_the_library(inputs):
    """A contiguous bf16 view at an odd element offset passes the binding's checks but is
    not 16-byte aligned: the library returns PFA_ERR_ALIGN and launches nothing."""
    from packed_varlen_flash_amd import PfaError, pfa_varlen_fwd
    wl, q, k, v, cu, torch = inputs
    T, H, d = q.shape
    buf = torch.empty(T * H * d + 8, dtype=torch.bfloat16, device="cuda")
    qv = buf[1:1 + T * H * d].view(T, H, d)
    qv.copy_(q)
    with pytest.raises(PfaError) as e:
        pfa_varlen_fwd(qv, k, v, cu, wl.max_seqlen, wl.scale)
    assert e.value.status == -12
    out = buf[1:1 + T * H * d].view(T, H, d)
    with pytest.raises(PfaError) as e:
        pfa_varlen_fwd(q, k, v, cu, wl.max_seqlen, wl.scale, out=out)
    assert e.value.status == -12
