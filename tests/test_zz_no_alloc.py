"""pfa_varlen_bwd_noalloc (row statistics in the library's own device array, no caller
workspace, nothing allocated) against pfa_varlen_bwd (caller workspace): the same kernels
run on the same inputs, so dq, dk and dv must be bitwise equal.  Two calls in a row, the
second on a smaller pack, so a stale array from the first call cannot go unnoticed; both
through the raw C ABI."""
import ctypes

import numpy as np
import pytest

import pfa_workloads as W
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _raw_noalloc(q, k, v, o, dout, lse, cu, wl, dq, dk, dv, stream):
    from packed_varlen_flash_amd import _lib
    P = ctypes.c_void_p
    return _lib.load().pfa_varlen_bwd_noalloc(
        P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(o.data_ptr()), P(dout.data_ptr()),
        P(lse.data_ptr()), P(cu.data_ptr()), len(wl.lengths), wl.max_seqlen, wl.total_tokens,
        wl.heads, wl.head_dim, wl.scale, P(dq.data_ptr()), P(dk.data_ptr()), P(dv.data_ptr()),
        P(stream.cuda_stream))


def _case(wl, seed):
    import torch
    from packed_varlen_flash_amd import pfa_varlen_bwd, pfa_varlen_fwd
    G.say(f"[gpu] noalloc backward vs workspace backward: {wl.name} T={wl.total_tokens} "
          f"H={wl.heads} d={wl.head_dim}")
    q, k, v, cu = G.upload(wl)
    o, lse = pfa_varlen_fwd(q, k, v, cu, wl.max_seqlen, wl.scale)
    rng = np.random.default_rng(seed)
    dout = G.to_dev(W.bf16_bits(rng.standard_normal(tuple(q.shape), dtype=np.float32)))
    ref = pfa_varlen_bwd(q, k, v, o, dout, lse, cu, wl.max_seqlen, wl.scale)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    stream = torch.cuda.current_stream()
    rc = _raw_noalloc(q, k, v, o, dout, lse, cu, wl, *got, stream)
    assert rc == 0, rc
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
    return got


def test_noalloc_backward_equals_workspace_backward_twice():
    big = W.make([1300, 700, 1, 2049, 64], 3, 128, seed=701, name="ragged d128")
    small = W.make([65, 300], 3, 128, seed=702, name="smaller pack d128")
    _case(big, 11)
    _case(small, 12)           # the array still holds the first call's (larger) statistics


def test_noalloc_backward_d64_and_capacity_check():
    import torch
    from packed_varlen_flash_amd import BWD_SCRATCH_FLOATS, PfaError, pfa_varlen_bwd_noalloc
    wl = W.make([513, 256, 77], 5, 64, seed=703, name="ragged d64")
    _case(wl, 13)
    # over capacity: rejected on the host, nothing launched
    heads = 2
    T = BWD_SCRATCH_FLOATS // (2 * heads) + 1
    q = torch.zeros((T, heads, 64), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    lse = torch.zeros((heads, T), device="cuda")
    with pytest.raises(PfaError) as e:
        pfa_varlen_bwd_noalloc(q, q, q, q, q, lse, cu, T, T)
    assert e.value.status == -11
