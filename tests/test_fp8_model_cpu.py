"""The statistical model of the FP8 P.V variant's error (tests/_fp8_model.py) against the
oracle's emulation of the variant's blocked steps, on the CPU.  The model uses only exact
softmax weights, the dequantised V and the variance of e4m3 rounding; the emulation rounds
every weight.  Agreement pins the model, which the GPU tests then apply to the kernel as a
check that does not depend on the emulation."""
import numpy as np
import pytest

import oracle
import pfa_workloads as W
from tests._fp8_model import E4M3_REL_VAR, predicted_rel_rms


def _case(lengths, heads, d, seed, q_mult=1.0):
    wl = W.make(lengths, heads, d, seed=seed)
    q = wl.q if q_mult == 1.0 else W.bf16_bits(W.bf16_to_f64(wl.q) * q_mult)
    codes, scales = oracle.quantize_v_fp8(wl.v, wl.cu_seqlens)
    vd = oracle.dequantize_v_fp8(codes, scales, wl.cu_seqlens)
    o_ex, _ = oracle.varlen_fwd(W.bf16_to_f64(q), W.bf16_to_f64(wl.k), vd, wl.cu_seqlens, wl.scale)
    return wl, q, codes, scales, vd, o_ex


def _rel(a, b):
    return float(np.sqrt(((a - b) ** 2).sum() / (b ** 2).sum()))


def test_rounding_variance_constant():
    # mean square relative error of round-to-nearest with 3 fraction bits over log-uniform
    # significands, by brute force over a fine grid of one binade
    x = np.exp2(np.linspace(0.0, 1.0, 2_000_001)[:-1])
    r = oracle.e4m3_round(x)
    assert abs(float(np.mean(((r - x) / x) ** 2)) / E4M3_REL_VAR - 1.0) < 2e-3


@pytest.mark.parametrize("lengths,heads,d,seed,q_mult", [
    ([900, 300, 64], 3, 128, 1, 1.0),
    ([512, 1, 777], 2, 64, 2, 1.0),
    ([2000], 2, 128, 3, 1.0),
    ([600, 257], 2, 128, 4, 3.0),     # sharper softmax: fewer weights carry the row
])
def test_model_matches_the_step_emulation(lengths, heads, d, seed, q_mult):
    wl, q, codes, scales, vd, o_ex = _case(lengths, heads, d, seed, q_mult)
    o_em, _ = oracle.varlen_fwd_fp8pv_blocked(q, wl.k, codes, scales, wl.cu_seqlens, wl.scale)
    ratio = _rel(o_em, o_ex) / predicted_rel_rms(q, wl.k, vd, wl.cu_seqlens, wl.scale, o_ex,
                                                 with_bf16=False)
    assert 0.9 <= ratio <= 1.1, ratio


def test_model_rejects_unrounded_weights():
    # the emulation with the rounding switched off is exact attention: the ratio collapses
    wl, q, codes, scales, vd, o_ex = _case([700, 300], 2, 128, 5)
    o_nq, _ = oracle.varlen_fwd_fp8pv_blocked(q, wl.k, codes, scales, wl.cu_seqlens, wl.scale,
                                              quantize=False)
    pred = predicted_rel_rms(q, wl.k, vd, wl.cu_seqlens, wl.scale, o_ex, with_bf16=False)
    assert _rel(o_nq, o_ex) / pred < 1e-6
