"""Pins of the acceptance checker ``oracle/compare.py`` (CPU only).

Every GPU parity verdict goes through four functions: ``lse_err``,
``loss_rel_err``, ``grad_errs`` and ``grad_ok``. They are pinned here against
values fixed by arithmetic alone (hand-computed maxima, cosines of parallel,
antiparallel and orthogonal vectors), against the stated tolerances (per-token
|lse - ref| <= 2e-3, mean-loss relative error <= 1e-4, max|x - ref| <=
1e-2 max|ref| with cosine >= 0.9999), and against planted mistakes: mutated
copies of the checker (a max over |x| instead of |ref|, a mean instead of a
max, a missing absolute value, reductions that skip NaN, a relative loss
error taken against the result, a cosine left unchecked) must each
give a different verdict on at least one of the cases below.
"""
import math

import numpy as np
import pytest

from oracle import compare as C


def test_tolerances_are_the_stated_ones():
    assert C.LSE_ABS == 2e-3
    assert C.LOSS_REL == 1e-4
    assert C.GRAD_MAXABS_REL == 1e-2
    assert C.GRAD_COS == 0.9999


# ---------------------------------------------------------------- lse_err

def test_lse_err_is_the_max_absolute_difference():
    assert C.lse_err([1.0, 2.0, 3.0], [1.0, 2.5, 2.75]) == 0.5
    assert C.lse_err([5.0], [5.0]) == 0.0
    assert C.lse_err([], []) == 0.0
    # sign of the difference does not matter
    assert C.lse_err([0.0, 0.0], [0.25, -0.375]) == 0.375


def _lse_accepts(lse, ref, err=C.lse_err):
    return err(lse, ref) <= C.LSE_ABS


def test_lse_rejects_one_token_over_tolerance():
    ref = np.linspace(3.0, 12.0, 65536)
    lse = ref.copy()
    assert _lse_accepts(lse, ref)
    lse[40000] += 2.1e-3          # one token just over the bound
    assert not _lse_accepts(lse, ref)
    lse[40000] = ref[40000] - 2.1e-3
    assert not _lse_accepts(lse, ref)
    lse[40000] = ref[40000] + 1.9e-3
    assert _lse_accepts(lse, ref)


def test_lse_rejects_nan_and_inf():
    ref = np.ones(100)
    for bad in (np.nan, np.inf, -np.inf):
        lse = ref.copy()
        lse[7] = bad
        assert not _lse_accepts(lse, ref)


def test_lse_planted_mistakes_are_caught():
    ref = np.linspace(3.0, 12.0, 1000)
    lse = ref.copy()
    lse[10] += 2.1e-3       # one bad token among many good ones
    lse[11] -= 1e-3

    def mean_err(a, b):      # mistake: mean instead of max
        return float(np.mean(np.abs(np.asarray(a) - np.asarray(b))))

    def signed_err(a, b):    # mistake: no absolute value
        return float(np.max(np.asarray(a) - np.asarray(b)))

    def nan_blind(a, b):     # mistake: NaN-ignoring max
        return float(np.nanmax(np.abs(np.asarray(a) - np.asarray(b))))

    assert not _lse_accepts(lse, ref)
    assert _lse_accepts(lse, ref, mean_err)
    neg = ref.copy()
    neg[3] -= 5e-3
    assert not _lse_accepts(neg, ref)
    assert _lse_accepts(neg, ref, signed_err)
    nan = ref.copy()
    nan[5] = np.nan
    assert not _lse_accepts(nan, ref)
    assert _lse_accepts(nan, ref, nan_blind)


# ---------------------------------------------------------------- loss

def test_loss_rel_err_values():
    assert C.loss_rel_err(10.001, 10.0) == pytest.approx(1e-4)
    assert C.loss_rel_err(-2.0, -2.5) == pytest.approx(0.2)
    # a zero reference (every token ignored) falls back to the absolute error
    assert C.loss_rel_err(0.0, 0.0) == 0.0
    assert C.loss_rel_err(3e-5, 0.0) == 3e-5


def test_loss_acceptance_edges():
    ref = 7.123456
    assert C.loss_rel_err(ref * (1 + 0.9e-4), ref) <= C.LOSS_REL
    assert not C.loss_rel_err(ref * (1 + 1.1e-4), ref) <= C.LOSS_REL
    assert not C.loss_rel_err(ref * (1 - 1.1e-4), ref) <= C.LOSS_REL
    assert not C.loss_rel_err(float("nan"), ref) <= C.LOSS_REL
    assert not C.loss_rel_err(float("inf"), ref) <= C.LOSS_REL


def test_loss_planted_mistake_relative_to_the_result():
    # mistake: dividing by |loss| instead of |ref| accepts a result that is
    # too large by slightly more than the bound
    def rel_to_x(x, ref):
        return abs(x - ref) / abs(x)

    ref = 1.0
    x = 1.0 + 1.00005e-4
    assert not C.loss_rel_err(x, ref) <= C.LOSS_REL
    assert rel_to_x(x, ref) <= C.LOSS_REL


# ---------------------------------------------------------------- gradients

def test_grad_errs_values():
    mabs, mref, cos = C.grad_errs([1.0, 2.0, -3.0], [1.0, 2.5, -3.0])
    assert (mabs, mref) == (0.5, 3.0)
    assert cos == pytest.approx((1 + 5 + 9) / math.sqrt(14 * 16.25))
    # parallel, antiparallel, orthogonal
    assert C.grad_errs([2.0, 0.0], [1.0, 0.0])[2] == pytest.approx(1.0)
    assert C.grad_errs([-1.0, 0.0], [1.0, 0.0])[2] == pytest.approx(-1.0)
    assert C.grad_errs([0.0, 1.0], [1.0, 0.0])[2] == pytest.approx(0.0)
    # both zero (all tokens ignored) agree exactly; one zero does not
    assert C.grad_errs(np.zeros(4), np.zeros(4)) == (0.0, 0.0, 1.0)
    assert C.grad_errs(np.zeros(4), np.ones(4))[2] == 0.0
    assert C.grad_errs(np.ones(4), np.zeros(4))[2] == 0.0
    # shape does not matter (the arrays are compared as flat vectors)
    a = np.arange(12.0).reshape(3, 4)
    assert C.grad_errs(a, a) == C.grad_errs(a.ravel(), a.ravel())


def _grad_case(seed=0, n=4096):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(n)


def test_grad_ok_accepts_small_noise():
    ref = _grad_case()
    x = ref + 1e-4 * _grad_case(1)
    ok, (mabs, mref, cos) = C.grad_ok(x, ref)
    assert ok and mabs < 1e-2 * mref and cos > 0.99999


def test_grad_ok_rejects_sign_flip_nan_and_zero():
    ref = _grad_case()
    assert not C.grad_ok(-ref, ref)[0]
    assert C.grad_ok(-ref, ref)[1][2] == pytest.approx(-1.0)
    for bad in (np.nan, np.inf):
        x = ref.copy()
        x[123] = bad
        assert not C.grad_ok(x, ref)[0]
    assert not C.grad_ok(np.zeros_like(ref), ref)[0]


def test_grad_ok_rejects_one_element_over_the_bound():
    ref = _grad_case()
    m = float(np.max(np.abs(ref)))
    j = int(np.argmax(np.abs(ref)))
    k = (j + 17) % ref.size
    x = ref.copy()
    x[k] += 1.05e-2 * m           # cosine stays above 0.9999
    ok, (mabs, mref, cos) = C.grad_ok(x, ref)
    assert cos >= C.GRAD_COS and mabs > C.GRAD_MAXABS_REL * mref
    assert not ok
    x[k] = ref[k] + 0.95e-2 * m
    assert C.grad_ok(x, ref)[0]


def test_grad_ok_rejects_low_cosine_with_small_max_error():
    # many elements each off by less than 1% of max|ref|: the max-error
    # test passes, the cosine does not
    ref = _grad_case()
    m = float(np.max(np.abs(ref)))
    x = ref + 0.009 * m * np.sign(_grad_case(2))
    ok, (mabs, mref, cos) = C.grad_ok(x, ref)
    assert mabs <= C.GRAD_MAXABS_REL * mref and cos < C.GRAD_COS
    assert not ok


def test_grad_planted_mistakes_are_caught():
    def errs_max_over_x(x, ref):     # mistake: scale by max|x|
        x = np.asarray(x, np.float64).ravel()
        ref = np.asarray(ref, np.float64).ravel()
        return (float(np.max(np.abs(x - ref))), float(np.max(np.abs(x))),
                C.grad_errs(x, ref)[2])

    def errs_no_cos(x, ref):         # mistake: the cosine is never checked
        mabs, mref, _ = C.grad_errs(x, ref)
        return mabs, mref, 1.0

    def errs_nan_blind(x, ref):      # mistake: NaN-ignoring reductions
        x = np.asarray(x, np.float64).ravel()
        ref = np.asarray(ref, np.float64).ravel()
        ok = np.isfinite(x)
        return (float(np.nanmax(np.abs(x - ref))), float(np.max(np.abs(ref))),
                float(np.dot(x[ok], ref[ok]) /
                      (np.linalg.norm(x[ok]) * np.linalg.norm(ref[ok]))))

    def verdict(errs, x, ref):
        mabs, mref, cos = errs(x, ref)
        return mabs <= C.GRAD_MAXABS_REL * mref and cos >= C.GRAD_COS

    ref = _grad_case()
    j = int(np.argmax(np.abs(ref)))
    m = abs(ref[j])
    # the largest element is too large by 1.005% of max|ref|: over the bound
    # against max|ref|, under it against max|x| (= 1.01005 max|ref|)
    x = ref.copy()
    x[j] += np.sign(ref[j]) * 1.005e-2 * m
    assert not C.grad_ok(x, ref)[0]
    assert verdict(errs_max_over_x, x, ref)
    low = ref + 0.009 * m * np.sign(_grad_case(2))
    assert not C.grad_ok(low, ref)[0]
    assert verdict(errs_no_cos, low, ref)
    y = ref.copy()
    y[5] = np.nan
    assert not C.grad_ok(y, ref)[0]
    assert verdict(errs_nan_blind, y, ref)


def test_report_formats_values():
    s = C.report("case", lse=1.5e-4, ok=True, n=3, bad=float("nan"))
    assert s == "[case] lse=1.500e-04 ok=True n=3 bad=nan"
