"""Pins of the expert-weight audit oracle (model-hub discussion "singular
matrices in Qwen3.8-2.4T-A95B": zero share and sigma_rob = 1.4826 * MAD):
hand-worked sets, rank-counting brute force on tiny sets, the normal
consistency of the scale, invariances, and the page's zero-majority case."""
import math

import numpy as np

from oracle import audit as oa


def brute_order_stat(vals, k):
    # the value x with #(v < x) <= k < #(v <= x): counting, no sorting
    for x in vals:
        below = sum(1 for v in vals if v < x)
        upto = sum(1 for v in vals if v <= x)
        if below <= k < upto:
            return x
    raise AssertionError("no order statistic")


def brute_median(vals):
    n = len(vals)
    if n % 2:
        return float(brute_order_stat(vals, n // 2))
    return (brute_order_stat(vals, n // 2 - 1) + brute_order_stat(vals, n // 2)) / 2.0


def test_hand_odd():
    r = oa.audit_values([3.0, -1.0, 0.0, 0.0, 5.0])
    # sorted -1 0 0 3 5 -> median 0; |w - 0| = 3 1 0 0 5 -> sorted 0 0 1 3 5 -> MAD 1
    assert r["median"] == 0.0 and r["mad"] == 1.0 and r["sigma_rob"] == 1.4826
    assert r["n_zero"] == 2 and r["n"] == 5 and r["zero_frac"] == 0.4


def test_hand_even():
    r = oa.audit_values([1.0, 2.0, 3.0, 10.0])
    # median (2 + 3) / 2 = 2.5; |w - 2.5| = 1.5 .5 .5 7.5 -> middle .5 and 1.5 -> MAD 1
    assert r["median"] == 2.5 and r["mad"] == 1.0 and r["sigma_rob"] == 1.4826
    assert r["n_zero"] == 0


def test_against_rank_counting_on_tiny_sets():
    rng = np.random.default_rng(0)
    for n in list(range(1, 12)) + [16, 31]:
        for _ in range(5):
            # few distinct values, so ties and duplicates are common
            vals = [float(v) for v in rng.integers(-4, 5, size=n) * 0.25]
            med = brute_median(vals)
            mad = brute_median([abs(v - med) for v in vals])
            r = oa.audit_values(vals)
            assert r["median"] == med and r["mad"] == mad
            assert r["n_zero"] == sum(1 for v in vals if v == 0)


def test_zero_majority_gives_zero_spread():
    # the page's case: with more than half of the entries exactly zero the
    # median is 0 and so is the median distance from it
    rng = np.random.default_rng(1)
    w = rng.normal(0, 0.02, size=100_000)
    w[rng.random(w.size) < 0.71] = 0.0
    r = oa.audit_values(w)
    assert r["median"] == 0.0 and r["mad"] == 0.0 and r["sigma_rob"] == 0.0
    assert abs(r["zero_frac"] - 0.71) < 0.01


def test_normal_consistency():
    # MAD of N(0, s) is s * Phi^-1(3/4), and 1.4826 * Phi^-1(3/4) = 1.00002
    q = math.sqrt(2.0) * 0.4769362762044699  # Phi^-1(3/4) = sqrt(2) erfinv(1/2)
    assert abs(1.4826 * q - 1.0) < 5e-5
    rng = np.random.default_rng(2)
    for s in (0.02, 1.0, 7.5):
        r = oa.audit_values(rng.normal(0.3, s, size=400_001))
        assert abs(r["sigma_rob"] / s - 1.0) < 0.012
        assert abs(r["median"] - 0.3) < 0.01 * s


def test_shift_scale_and_order_invariance():
    rng = np.random.default_rng(3)
    w = np.round(rng.normal(0, 1, size=1001) * 64) / 64  # dyadic, so shifts and doublings are exact
    r = oa.audit_values(w)
    rs = oa.audit_values(w + 3.0)
    assert rs["median"] == r["median"] + 3.0 and rs["mad"] == r["mad"]
    r2 = oa.audit_values(w * 2.0)
    assert r2["median"] == 2 * r["median"] and r2["mad"] == 2 * r["mad"]
    rn = oa.audit_values(-w)
    assert rn["median"] == -r["median"] and rn["mad"] == r["mad"]
    rp = oa.audit_values(rng.permutation(w))
    assert rp == r


def test_signed_zeros_nan_and_empty():
    r = oa.audit_values([-0.0, 0.0, -0.0, 1.0])
    assert r["n_zero"] == 3 and r["median"] == 0.0
    r = oa.audit_values([1.0, float("nan"), 2.0])
    assert r["n_nan"] == 1 and math.isnan(r["median"]) and math.isnan(r["sigma_rob"])
    r = oa.audit_values([])
    assert r["n"] == 0 and math.isnan(r["median"])


def test_slices_and_whole():
    rng = np.random.default_rng(4)
    w = rng.normal(0, 1, size=(3, 5, 7))
    per, whole = oa.audit(w, 3)
    assert len(per) == 3 and whole["n"] == 105
    for s in range(3):
        assert per[s]["median"] == brute_median(list(w[s].reshape(-1)))
    assert whole["median"] == brute_median(list(w.reshape(-1)))
