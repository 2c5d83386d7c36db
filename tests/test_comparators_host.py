"""The GPU tests' comparators reject what they must (CPU only).

Every oracle comparison of the GPU suite goes through these helpers, so a
comparator that lets a NaN, an infinity or an out-of-bound value through
would make every such test pass vacuously.  Each case below plants one bad
element in an otherwise exact result.
"""

from __future__ import annotations

import numpy as np
import pytest

from seer_testlib import assert_gt_close, assert_lse_close, assert_out_close


def _ref(shape=(4, 16), seed=0):
    return np.random.default_rng(seed).normal(size=shape)


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf, "far"])
@pytest.mark.parametrize("helper", [assert_out_close, assert_gt_close])
def test_output_comparators_reject_one_bad_element(helper, bad):
    ref = np.abs(_ref()) if helper is assert_gt_close else _ref()
    got = ref.copy()
    got[2, 5] = ref[2, 5] + 1.0 if bad == "far" else bad
    with pytest.raises(AssertionError):
        helper(got, ref, "planted")


@pytest.mark.parametrize("helper", [assert_out_close, assert_gt_close])
def test_output_comparators_accept_in_bound_values(helper):
    ref = np.abs(_ref()) if helper is assert_gt_close else _ref()
    # just inside each bound: out 2e-2 + 1e-2|ref|, ground truth 1e-6 + 2e-3|ref|
    slack = (2e-2 + 1e-2 * np.abs(ref) if helper is assert_out_close
             else 1e-6 + 2e-3 * np.abs(ref))
    helper(ref + 0.99 * slack, ref, "inside")
    helper(ref - 0.99 * slack, ref, "inside")


def test_output_comparators_reject_a_shape_mismatch():
    ref = _ref()
    with pytest.raises(AssertionError):
        assert_out_close(ref[:, :8], ref, "shape")
    with pytest.raises(AssertionError):
        assert_gt_close(np.abs(ref)[:3], np.abs(ref), "shape")


@pytest.mark.parametrize("bad", [np.nan, np.inf, 1.0])
def test_lse_comparator_rejects_one_bad_element(bad):
    ref = _ref((8,))
    got = ref.copy()
    got[3] = ref[3] + bad if bad == 1.0 else bad
    with pytest.raises(AssertionError):
        assert_lse_close(got, ref, "planted")


def test_lse_comparator_matches_empty_selections_only_to_minus_inf():
    ref = _ref((8,))
    ref[1] = -np.inf
    got = ref.copy()
    assert_lse_close(got, ref, "both -inf")
    got[1] = 0.0
    with pytest.raises(AssertionError):
        assert_lse_close(got, ref, "finite against -inf")
    got = ref.copy()
    got[4] = -np.inf
    with pytest.raises(AssertionError):
        assert_lse_close(got, ref, "-inf against finite")
