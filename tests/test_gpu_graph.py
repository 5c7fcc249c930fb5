"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph): every replay must
equal the eager result bit for bit, with eager work and synchronisation between replays.
The calls allocate nothing and launch only kernels on the caller's stream, so they can be
captured as they are."""
import numpy as np
import pytest

import pfa_workloads as W
from tests._gpu import say, to_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy()
    if t.dtype == torch.float32:
        return t.contiguous().view(torch.int32).cpu().numpy()
    return t.contiguous().cpu().numpy()


def _check_graph(label, run, outputs, reset):
    """run() launches the calls into outputs; reset() scribbles over them."""
    import torch
    say(f"[gpu] graph capture {label}")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                                   # warm-up outside capture (first-call setup)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = [_bits(t) for t in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(outputs, eager):
            np.testing.assert_array_equal(_bits(t), e, err_msg=f"{label}: replay {rep}")
        x = torch.randn(1 << 20, device="cuda")            # eager work between replays
        (x * 2).sum().item()


def test_forward_and_backward_in_a_graph():
    import torch
    from packed_varlen_flash_amd import pfa_varlen_bwd, pfa_varlen_fwd
    wl = W.make([1024, 1, 300, 0, 700], 4, 128, seed=600)
    q, k, v = to_dev(wl.q), to_dev(wl.k), to_dev(wl.v)
    do = to_dev(W.bf16_bits(np.random.default_rng(601).standard_normal(wl.q.shape, dtype=np.float32)))
    cu = torch.from_numpy(wl.cu_seqlens).to("cuda")
    out, lse = torch.empty_like(q), torch.empty((wl.heads, wl.total_tokens), device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty((2, wl.heads, wl.total_tokens), device="cuda")
    stream = lambda: torch.cuda.current_stream()

    def run():
        pfa_varlen_fwd(q, k, v, cu, wl.max_seqlen, wl.scale, out=out, lse=lse, stream=stream())
        pfa_varlen_bwd(q, k, v, out, do, lse, cu, wl.max_seqlen, wl.scale, dq=dq, dk=dk, dv=dv,
                       workspace=ws, stream=stream())

    def reset():
        for t in (out, dq, dk, dv):
            t.fill_(float("nan"))
        lse.fill_(float("nan"))
    _check_graph("forward + backward", run, [out, lse, dq, dk, dv], reset)


def test_fp8_quantiser_and_forward_in_a_graph():
    import torch
    from packed_varlen_flash_amd import pfa_quantize_v_fp8, pfa_varlen_fwd_fp8pv
    wl = W.make([513, 64, 900], 2, 128, seed=602)
    q, k, v = to_dev(wl.q), to_dev(wl.k), to_dev(wl.v)
    cu = torch.from_numpy(wl.cu_seqlens).to("cuda")
    v8 = torch.empty((wl.total_tokens, 2, 128), dtype=torch.uint8, device="cuda")
    vs = torch.empty((3, 2, 128), dtype=torch.float32, device="cuda")
    out, lse = torch.empty_like(q), torch.empty((2, wl.total_tokens), device="cuda")

    def run():
        s = torch.cuda.current_stream()
        pfa_quantize_v_fp8(v, cu, v8=v8, v_scale=vs, stream=s)
        pfa_varlen_fwd_fp8pv(q, k, v8, vs, cu, wl.max_seqlen, wl.scale, out=out, lse=lse, stream=s)

    def reset():
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        v8.fill_(0x7F)
        vs.fill_(float("nan"))
    _check_graph("fp8 quantiser + forward", run, [out, lse, v8, vs], reset)
