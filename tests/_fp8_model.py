"""A statistical model of the FP8 P.V variant's error, independent of any emulation of its
steps: the expected relative RMS of O_fp8 - O, where O is exact attention on the
dequantised V and the difference comes from rounding each weight to e4m3.

The variant forms weights w_j = 2^8 2^(s_j log2(e) - m) against the running maximum m of
the keys visited so far (64-key blocks in order), rounds each w_j to the nearest e4m3
number, and divides by the unrounded sum of the w_j (GigaPath-Flash page, section 3.2, for
the blocked update; the FP8 step is the variant's own).  Relative to the final maximum
that is O_fp8 = sum_j (1 + e_j) p_j V_j / sum_j p_j with p_j = exp(s_j - max) and e_j the
relative rounding error of w_j, so

    E |O_fp8 - O|^2 (per element c) = sum_j E[e_j^2] p_j^2 V_jc^2 / (sum_j p_j)^2

for independent, zero-mean e_j (round to nearest).  A key whose score equals the running
maximum of its block has w_j = 2^8 exactly: e_j = 0.  For any other weight the fractional
part of log2 w_j is spread over [0, 1), i.e. w_j is log-uniform within its binade.  With 3
fraction bits the grid on [1, 2) is g_k = 1 + k/8, and
E[e_j^2] = (1 / ln 2) sum_k int over g_k's rounding cell of (x - g_k)^2 / x^3 dx
= 7.02e-4 (about 2^-6 / 12 times E[1 / x^2]).  (Weights below 2^-6, e4m3's subnormal range,
belong to keys 2^-14 below the maximum and are left out.)  The bf16 rounding of the output
adds an independent ulp^2 / 12 per element.
"""
import math

import numpy as np

import pfa_workloads as W


def _e4m3_rel_var():
    # antiderivative of (x - g)^2 / x^3 = 1/x - 2g/x^2 + g^2/x^3
    F = lambda x, g: math.log(x) + 2.0 * g / x - g * g / (2.0 * x * x)
    total = 0.0
    for k in range(9):
        g = 1.0 + k / 8.0
        a, b = max(1.0, g - 1.0 / 16.0), min(2.0, g + 1.0 / 16.0)
        if b > a:
            total += F(b, g) - F(a, g)
    return total / math.log(2.0)


E4M3_REL_VAR = _e4m3_rel_var()


def bf16_rounding_var(o):
    """ulp^2 / 12 of bf16 (8 significant bits) at |o|: the variance of round-to-nearest."""
    ao = np.maximum(np.abs(o), np.finfo(np.float32).tiny)
    ulp = np.ldexp(1.0, np.floor(np.log2(ao)).astype(np.int64) - 7)
    return ulp * ulp / 12.0


def predicted_sq_error(q_bits, k_bits, vd, cu_seqlens, scale, rows=None, block=64):
    """Expected squared error sum over [rows, H, d] from the weight rounding alone (fp64)."""
    q, k = W.bf16_to_f64(q_bits), W.bf16_to_f64(k_bits)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, d = q.shape
    want = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    seg = np.searchsorted(cu[1:], want, side="right")
    total = 0.0
    for s in sorted(set(seg.tolist())):
        a, b = int(cu[s]), int(cu[s + 1])
        if b <= a:
            continue
        qi = want[seg == s]
        starts = np.arange(0, b - a, block)
        for h in range(H):
            sc = (q[qi, h] @ k[a:b, h].T) * scale                 # [n, L]
            p = np.exp(sc - sc.max(axis=1, keepdims=True))
            # running maximum over whole blocks, broadcast back to each key
            run = np.maximum.accumulate(np.maximum.reduceat(sc, starts, axis=1), axis=1)
            run_key = np.repeat(run, np.diff(np.append(starts, b - a)), axis=1)
            var = np.where(sc == run_key, 0.0, E4M3_REL_VAR) * p * p
            num = var @ (vd[a:b, h] ** 2)                          # [n, d]
            total += float((num / (p.sum(axis=1, keepdims=True) ** 2)).sum())
    return total


def predicted_rel_rms(q_bits, k_bits, vd, cu_seqlens, scale, o_exact, rows=None, with_bf16=True):
    """Expected relative RMS of the variant's output against o_exact (exact attention on the
    dequantised V, [rows, H, d]): weight rounding, plus the bf16 output rounding if asked."""
    sq = predicted_sq_error(q_bits, k_bits, vd, cu_seqlens, scale, rows=rows)
    if with_bf16:
        sq += float(bf16_rounding_var(o_exact).sum())
    return math.sqrt(sq / float((o_exact ** 2).sum()))
