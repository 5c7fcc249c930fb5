"""Helpers for GPU parity tests: upload seeded inputs, run the HIP path, compare."""
import sys

import numpy as np

import pfa_workloads as W

# Bars for bf16 inputs against the fp64 oracle: max |err| and relative RMS of the output,
# max |err| of the LSE (see the rounding note at compare()).
MAX_ABS = 1e-2
REL_RMS = 4e-3
LSE_ABS = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def from_dev_bf16(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def upload(wl):
    import torch
    return (to_dev(wl.q), to_dev(wl.k), to_dev(wl.v),
            torch.from_numpy(wl.cu_seqlens.astype(np.int32)).to("cuda"))


def run(wl, label="", want_lse=True, dev=None, stream=None):
    """Run pfa_varlen_fwd on a Workload; returns (out bits [T,H,d] uint16, lse [H,T] f32)."""
    import torch
    from packed_varlen_flash_amd import pfa_varlen_fwd
    say(f"[gpu] pfa_varlen_fwd {label or wl.name}: segs={len(wl.lengths)} T={wl.total_tokens} "
        f"H={wl.heads} d={wl.head_dim} max_seqlen={wl.max_seqlen}")
    q, k, v, cu = dev if dev is not None else upload(wl)
    out, lse = pfa_varlen_fwd(q, k, v, cu, wl.max_seqlen, wl.scale, want_lse=want_lse, stream=stream)
    torch.cuda.synchronize()
    return from_dev_bf16(out), (lse.cpu().numpy() if lse is not None else None)


def bf16_half_ulp(x):
    """Half the spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.ldexp(1.0, np.floor(np.log2(ax)).astype(np.int64) - 8)


# The 1e-2 bar leaves 1e-2 - 2^-7 for the kernel's own error at |O| in [2, 4), where bf16
# rounding of the output alone can take 2^-7.  At |O| >= 4 rounding alone can exceed the
# bar, so there the bound is that element's own rounding step plus the same allowance.
KERNEL_ALLOWANCE = MAX_ABS - 2.0 ** -7


def compare(out_bits, lse, o_ref, l_ref):
    o = W.bf16_to_f64(out_bits)
    diff = o - o_ref
    ad = np.abs(diff)
    big = np.abs(o_ref) >= 4.0
    max_abs = float(ad.max()) if diff.size else 0.0
    max_abs_small = float(ad[~big].max()) if np.any(~big) else 0.0
    excess_big = float((ad[big] - bf16_half_ulp(o_ref[big])).max()) if np.any(big) else -1.0
    denom = float(np.sqrt(np.sum(o_ref * o_ref)))
    rel_rms = float(np.sqrt(np.sum(diff * diff)) / denom) if denom > 0 else 0.0
    lse_abs = float(np.abs(lse.astype(np.float64) - l_ref).max()) if lse is not None and lse.size else 0.0
    # elements over the raw 1e-2 bar: they can pass only through the |O_ref| >= 4 allowance
    n_over = int(np.count_nonzero(ad > MAX_ABS))
    return dict(max_abs=max_abs, max_abs_small=max_abs_small, excess_big=excess_big,
                rel_rms=rel_rms, lse_abs=lse_abs, n_big=int(big.sum()), n_over_raw_bar=n_over)


def assert_parity(m, label=""):
    """Raw max|err| is printed against the 1e-2 bar as written; elements over it pass only
    where |O_ref| >= 4 (bf16 rounding of the output alone can exceed 1e-2 there), and their
    count is printed too, so a pass through the allowance is visible in the log."""
    say(f"[parity] {label}: raw max|err|={m['max_abs']:.3e} (bar 1e-2; "
        f"{m.get('n_over_raw_bar', 0)} elements over it, passing only via the |O_ref|>=4 allowance) "
        f"(|O_ref|<4: {m['max_abs_small']:.3e}; "
        f"{m['n_big']} elements >=4, worst excess over rounding {m['excess_big']:.3e}) "
        f"relRMS={m['rel_rms']:.3e} LSE={m['lse_abs']:.3e}")
    assert m["max_abs_small"] <= MAX_ABS, m
    assert m["excess_big"] <= KERNEL_ALLOWANCE, m
    assert m["rel_rms"] <= REL_RMS, m
    assert m["lse_abs"] <= LSE_ABS, m
