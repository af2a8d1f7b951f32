"""Pins of the parity criterion itself (oracle/tolerance.py), on the CPU.

The criterion reads the bar "max|err| <= 2e-2 rms(ref), per-element relative
error <= 5e-2 where |ref| > rms" elementwise: an element with |ref| <= rms
passes when |err| <= 2e-2 rms, one with |ref| > rms when |err| <= 5e-2 |ref|.
Each case sits just inside or just outside one clause, so that a loosened or
tightened constant, a swapped clause, a >= for the strict > in the large test,
a rms taken over the wrong values, or NaN passing, fails one of them."""
import numpy as np
import pytest

from oracle import tolerance


def small_ref():
    # |ref| = 1 everywhere: rms(ref) = 1 exactly and every element is "small"
    return np.array([1.0, -1.0, 1.0, -1.0] * 16)


def test_constants():
    assert tolerance.ABS_REL_RMS == 2e-2 and tolerance.REL_LARGE == 5e-2


@pytest.mark.parametrize("delta,ok", [(0.0199, True), (-0.0199, True), (0.0201, False),
                                      (-0.0201, False)])
def test_small_clause_boundary(delta, ok):
    ref = small_ref()
    out = ref.copy()
    out[5] += delta
    res = tolerance.check(out, ref)
    assert res["ok"] is ok, res
    assert res["n_bad"] == (0 if ok else 1)
    assert np.isclose(res["rms"], 1.0)
    assert np.isclose(res["max_small_err_over_rms"], abs(delta))


def large_ref():
    # one large element (|ref| = 3) among small ones: rms = sqrt((9 + 63 * 0.01) / 64)
    ref = np.full(64, 0.1)
    ref[7] = 3.0
    return ref


@pytest.mark.parametrize("rel,ok", [(0.0499, True), (0.0501, False)])
def test_large_clause_boundary(rel, ok):
    ref = large_ref()
    rms = float(np.sqrt(np.mean(ref * ref)))
    assert abs(ref[7]) > rms and np.all(np.abs(np.delete(ref, 7)) <= rms)
    out = ref.copy()
    out[7] = ref[7] * (1 + rel)
    res = tolerance.check(out, ref)
    assert res["ok"] is ok, res
    assert np.isclose(res["max_large_rel"], rel)
    # this error is far above 2e-2 rms: only the large-element clause lets it pass
    assert abs(out[7] - ref[7]) > 2e-2 * rms


def test_large_clause_does_not_cover_small_elements():
    # the same relative error on a small element fails (its limit is 2e-2 rms)
    ref = large_ref()
    rms = float(np.sqrt(np.mean(ref * ref)))
    out = ref.copy()
    out[0] = ref[0] + 2.5e-2 * rms
    assert abs(out[0] - ref[0]) <= 5e-2 * max(abs(ref[0]), rms)
    assert not tolerance.check(out, ref)["ok"]


def test_element_equal_to_rms_is_small():
    # |ref| == rms exactly takes the small clause (the large test is strict):
    # an error between 2e-2 rms and 5e-2 |ref| must fail
    ref = small_ref()
    out = ref.copy()
    out[3] += 0.03 * np.sign(ref[3])
    assert not tolerance.check(out, ref)["ok"]


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_non_finite_outputs_fail(bad):
    ref = small_ref()
    out = ref.copy()
    out[2] = bad
    res = tolerance.check(out, ref)
    assert not res["ok"] and res["n_bad"] == 1


def test_rms_is_over_all_checked_elements():
    # scaling ref and out together leaves the verdict unchanged; doubling only
    # the large element changes the small elements' limit through rms
    ref = large_ref()
    out = ref + 0.02 * 0.9 * np.sqrt(np.mean(ref * ref))
    assert tolerance.check(out, ref)["ok"]
    assert tolerance.check(4 * out, 4 * ref)["ok"]
    ref2 = ref.copy()
    ref2[7] = 1.0  # smaller rms: the same absolute errors now exceed 2e-2 rms
    out2 = out.copy()
    out2[7] = 1.0
    assert not tolerance.check(out2, ref2)["ok"]


def test_all_small_and_zero_reference():
    # every |ref| equal (none exceeds rms): only the small clause applies
    ref = small_ref()
    assert tolerance.check(ref * (1 + 0.019), ref)["ok"]
    assert not tolerance.check(ref * (1 + 0.021), ref)["ok"]
    # an all-zero reference has rms 0: only an exact output passes
    z = np.zeros(8)
    assert tolerance.check(z, z)["ok"]
    out = z.copy()
    out[1] = 1e-30
    assert not tolerance.check(out, z)["ok"]


def test_shape_mismatch_is_an_error():
    with pytest.raises(AssertionError):
        tolerance.check(np.zeros(3), np.zeros(4))
