"""The GPU tests' comparison helpers, checked on the CPU with planted
differences: each must accept what the method allows and reject the rest.

- check_routing: a selection that differs from the oracle's only across a
  near-tie (< 1e-6 in the FP64 logits) is accepted and reported; any other
  difference, a repeated expert or a routing weight off by more than 1e-6
  fails.
- mx_u_ties: a quantised u element that differs from the MX rounding of the
  exact u is accepted only when the kernel's own FP32 u lies within its
  formation bound and the kernel's code is the MX rounding of that FP32 value
  (a rounding midpoint between the two values).
- _check_f16: stored FP16 values one unit in the last place apart pass, two
  apart fail.
"""
import numpy as np
import pytest

from layer_cases import _check_f16, check_routing, mx_u_ties
from oracle import mx
from oracle import oracle as orc


def routed(logits, k):
    ids, _ = orc.select_topk(logits, k)
    return ids, orc.softmax_selected(logits, ids)


def test_routing_exact_and_near_tie():
    lg = np.array([[0.3, 1.2, -0.4, 0.9, 0.9 + 5e-7, -1.0]])
    ids, w = routed(lg, 2)
    assert ids.tolist() == [[1, 4]]
    near, _ = check_routing(ids.astype(np.int32), w.astype(np.float32), lg, 2)
    assert near == []
    # the GPU took expert 3 for slot 2: 5e-7 below expert 4, a near-tie
    gpu = np.array([[1, 3]], np.int32)
    sel = np.take_along_axis(lg, gpu.astype(np.int64), axis=1)
    gw = np.exp(sel - sel.max(1, keepdims=True))
    gw /= gw.sum(1, keepdims=True)
    near, _ = check_routing(gpu, gw.astype(np.float32), lg, 2)
    assert near == [0]


def test_routing_rejects_other_differences():
    lg = np.array([[0.3, 1.2, -0.4, 0.9, 0.95, -1.0]])
    ids, w = routed(lg, 2)
    with pytest.raises(AssertionError):  # expert 3 is 0.05 below expert 4: not a near-tie
        check_routing(np.array([[1, 3]], np.int32), w.astype(np.float32), lg, 2)
    with pytest.raises(AssertionError):  # the same expert twice
        check_routing(np.array([[1, 1]], np.int32), w.astype(np.float32), lg, 2)
    with pytest.raises(AssertionError):  # a weight off by 1e-5
        check_routing(ids.astype(np.int32), (w + np.array([[1e-5, -1e-5]])).astype(np.float32), lg, 2)


class _R:  # the oracle fields mx_u_ties reads
    def __init__(self, u_pre, u):
        self.u_pre, self.u = u_pre, u


def _tie_case():
    """One MX FP4 block (scale 1: amax 4): the exact u has 2.5 + 1e-7 (above
    the midpoint of the codes 2 and 3: rounds to 3), the kernel's FP32 u has
    2.5 exactly (the midpoint: rounds to the even code, 2)."""
    u_exact = np.zeros((1, 32))
    u_exact[0, 0] = 4.0
    u_exact[0, 1] = 2.5 + 1e-7
    u_exact[0, 2:] = 0.75
    pooled = u_exact.astype(np.float32)  # the kernel's gamma_p * h ...
    pooled[0, 1] = np.float32(2.5)
    v = {"pooled": pooled, "row_scale": np.ones(1, np.float32)}  # ... times a row scale of 1
    r = _R(u_exact, mx.quantize_mx(u_exact, "mxfp4")[0])
    return v, r


def test_mx_tie_across_a_midpoint_is_accepted():
    v, r = _tie_case()
    assert r.u[0, 1] == 3.0
    uq_gpu = mx.quantize_mx(v["pooled"].astype(np.float64), "mxfp4")[0]
    assert uq_gpu[0, 1] == 2.0
    ties, nel = mx_u_ties(v, np.arange(1), uq_gpu, r, "mxfp4")
    assert nel == 1 and list(ties) == [0] and np.array_equal(ties[0], uq_gpu[0])


def test_mx_codes_that_are_not_a_rounding_of_the_kernel_u_fail():
    v, r = _tie_case()
    uq_gpu = mx.quantize_mx(v["pooled"].astype(np.float64), "mxfp4")[0]
    bad = uq_gpu.copy()
    bad[0, 5] = 0.5  # 0.75 is the midpoint of 0.5 and 1.0 and rounds to the even code, 1.0
    with pytest.raises(AssertionError):
        mx_u_ties(v, np.arange(1), bad, r, "mxfp4")


def test_mx_kernel_u_outside_its_formation_bound_fails():
    v, r = _tie_case()
    v["pooled"] = v["pooled"].copy()
    v["pooled"][0, 3] = np.float32(0.76)  # 0.01 from the exact 0.75: far beyond FP32 formation error
    uq_gpu = mx.quantize_mx(v["pooled"].astype(np.float64), "mxfp4")[0]
    with pytest.raises(AssertionError):
        mx_u_ties(v, np.arange(1), uq_gpu, r, "mxfp4")


def test_f16_stage_check_allows_one_ulp():
    ref = np.array([1.0, 3.0, -0.125, 1000.0])
    ulp = np.array([2.0 ** -10, 2.0 ** -9, 2.0 ** -13, 0.5])
    assert _check_f16(ref + ulp, ref, 1.0, 0.0, "one ulp") == 1.0
    with pytest.raises(AssertionError):
        _check_f16(ref + 2 * ulp, ref, 1.0, 0.0, "two ulps")
    # stored times a power of two: the unit is that of the stored value (the
    # same relative step), so one unit still passes and two still fail
    assert _check_f16(ref + ulp, ref, 0.25, 0.0, "scaled") == 1.0
    with pytest.raises(AssertionError):
        _check_f16(ref + 2 * ulp, ref, 0.25, 0.0, "scaled, two ulps")
