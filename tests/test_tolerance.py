"""The parity comparison itself: bf16 output rounding is never charged to the kernel,
while a kernel error above the allowance is caught (CPU only)."""
import numpy as np

import pfa_workloads as W
from tests import _gpu as G


def _bits(x):
    return W.bf16_bits(np.asarray(x, np.float32))


def test_pure_output_rounding_passes():
    rng = np.random.default_rng(0)
    ref = rng.uniform(-7.9, 7.9, size=(400, 2, 8))
    m = G.compare(_bits(ref), None, ref, None)
    G.assert_parity(m, "rounding only")
    assert m["n_big"] > 0 and m["max_abs"] > G.MAX_ABS   # rounding alone exceeds 1e-2 at |O|>=4


def test_kernel_error_is_caught():
    ref = np.full((4, 1, 8), 3.0)
    m = G.compare(_bits(ref + 0.011), None, ref, None)
    assert m["max_abs_small"] > G.MAX_ABS
    ref_big = np.full((4, 1, 8), 5.0)
    m = G.compare(_bits(ref_big + 0.03), None, ref_big, None)
    assert m["excess_big"] > G.KERNEL_ALLOWANCE


def test_half_ulp():
    assert G.bf16_half_ulp(np.array([1.0]))[0] == 2.0 ** -8
    assert G.bf16_half_ulp(np.array([-4.0]))[0] == 2.0 ** -6
