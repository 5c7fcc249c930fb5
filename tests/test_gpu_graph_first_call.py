"""The library's very first call in a process made inside a HIP graph capture.

The library keeps per-device caches (compute-unit count, occupancy per kernel variant) and
fills them, with hipFuncSetAttribute and an occupancy query, on the first call that needs
them.  A caller may make that first call under stream capture.  The call must then either
be captured correctly (every replay equal to the eager result bit for bit) or fail with a
status code, after which eager calls still work.  Each case runs in a fresh child process,
so no earlier call has filled the caches."""
import os
import subprocess
import sys

import pytest

from tests._gpu import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, ROOT)
import pfa_workloads as W
from packed_varlen_flash_amd import PfaError, pfa_varlen_fwd, pfa_varlen_fwd_qk

CASE = sys.argv[1]
dev = torch.device("cuda:0")
up = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
if CASE == "self":
    x = W.make([700, 1, 300, 0, 1024], 4, 128, seed=610)
    q, k, v = up(x.q), up(x.k), up(x.v)
    cu = torch.from_numpy(x.cu_seqlens).to(dev)
    call = lambda o, l: pfa_varlen_fwd(q, k, v, cu, x.max_seqlen, x.scale, out=o, lse=l)
    T, H = x.total_tokens, x.heads
else:   # short key segments: the resident K/V kernel, d = 64
    x = W.make_cross([900, 1, 300, 64], [128, 0, 77, 5], 3, 64, seed=611, name="graph-first")
    q, k, v = up(x.q), up(x.k), up(x.v)
    cq, ck = torch.from_numpy(x.cu_q).to(dev), torch.from_numpy(x.cu_k).to(dev)
    call = lambda o, l: pfa_varlen_fwd_qk(q, k, v, cq, ck, x.max_q, x.max_k, x.scale, out=o, lse=l)
    T, H = x.total_q, x.heads
out, lse = torch.empty_like(q), torch.empty((H, T), dtype=torch.float32, device=dev)
torch.cuda.synchronize()
print("first library call inside capture:", CASE, flush=True)
g = torch.cuda.CUDAGraph()
status = "captured"
try:
    with torch.cuda.graph(g):
        call(out, lse)
except PfaError as e:
    status = f"status {e.status}"
except RuntimeError as e:
    status = f"capture ended with an error: {e}"
print("capture:", status, flush=True)
torch.cuda.synchronize()
ref_o, ref_l = torch.empty_like(out), torch.empty_like(lse)
call(ref_o, ref_l)                      # eager, after the capture
torch.cuda.synchronize()
assert torch.isfinite(ref_o.float()).all().item()
if status == "captured":
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), rep
        assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)), rep
        y = torch.randn(1 << 20, device=dev)          # eager work between replays
        (y * 2).sum().item()
print("OK", status, flush=True)
"""


@pytest.mark.parametrize("case", ["self", "resident"])
def test_first_library_call_inside_a_graph_capture(case):
    say(f"[gpu] first library call inside a graph capture ({case}), child process")
    script = _CHILD.replace("ROOT", repr(ROOT), 1)
    res = subprocess.run([sys.executable, "-c", script, case], capture_output=True, text=True,
                         timeout=240, cwd=ROOT)
    say(res.stdout.strip())
    assert res.returncode == 0, res.stdout + res.stderr
    last = res.stdout.strip().splitlines()[-1]
    assert last.startswith("OK "), res.stdout
