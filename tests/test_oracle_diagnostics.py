"""Pins of the mismatch-diagnostics oracle (oracle/diagnostics.py) against
what mathematics fixes independently of its code: closed forms, the exact KL
of two known categorical distributions (Monte Carlo), hand-sorted medians,
the telescoping split and bit-level counting."""

import math

import numpy as np
import pytest

import oracle

LN2 = math.log(2.0)


def test_ln2_shift_gives_weight_two():
    """delta = ln 2 everywhere: w = 2, |w - 1| = 1, k3 = 2 - 1 - ln 2."""
    lr = np.array([-3.0, -0.5, -7.25, -1.0])
    s = oracle.mismatch_stats(lr + LN2, lr)
    assert s["n_tok"] == 4
    assert abs(s["kl_k1"] + LN2) <= 1e-15
    assert abs(s["kl_k2"] - LN2 * LN2 / 2) <= 1e-15
    assert abs(s["kl_k3"] - (1.0 - LN2)) <= 1e-15
    assert abs(s["weight_mean"] - 2.0) <= 1e-15 and abs(s["weight_max"] - 2.0) <= 1e-15
    assert abs(s["deviation_max"] - 1.0) <= 1e-15 and abs(s["deviation_median"] - 1.0) <= 1e-15
    assert s["deviation_peak_over_median"] == pytest.approx(1.0, abs=1e-15)


def test_zero_lag_is_exactly_zero():
    lp = np.random.default_rng(1).normal(-2, 1, 1001).astype(np.float32)
    s = oracle.mismatch_stats(lp, lp.copy(), lp.copy())
    for k in ("kl_k1", "kl_k2", "kl_k3", "deviation_max", "deviation_median", "lag_abs_max", "kernel_abs_max",
              "kernel_nonzero", "lag_kl_k3", "kernel_kl_k3"):
        assert s[k] == 0.0, k
    assert s["weight_mean"] == 1.0 and s["weight_min"] == 1.0 and s["weight_max"] == 1.0
    assert s["deviation_peak_over_median"] == 1.0


@pytest.mark.parametrize("seed", [0, 1])
def test_k1_k3_unbiased_for_rollout_to_learner_kl(seed):
    """Tokens drawn from the rollout policy p = (0.9, 0.1); the learner's is
    q = (0.5, 0.5). E[k1] = E[k3] = KL(p || q) = 0.9 ln 1.8 + 0.1 ln 0.2
    exactly; the sample means must land within 5 standard errors. The
    reverse direction KL(q || p) = 0.5 ln(5/9) + 0.5 ln 5 and a flipped sign
    both miss by more than 100 standard errors."""
    rng = np.random.default_rng(seed)
    p = np.array([0.9, 0.1])
    q = np.array([0.5, 0.5])
    n = 400_000
    y = rng.choice(2, size=n, p=p)
    lr, lp = np.log(p)[y], np.log(q)[y]
    s = oracle.mismatch_stats(lp, lr)
    kl_pq = 0.9 * math.log(1.8) + 0.1 * math.log(0.2)
    kl_qp = 0.5 * math.log(5.0 / 9.0) + 0.5 * math.log(5.0)
    d = lp - lr
    se1 = np.std(-d) / math.sqrt(n)
    se3 = np.std(np.expm1(d) - d) / math.sqrt(n)
    assert abs(s["kl_k1"] - kl_pq) <= 5 * se1
    assert abs(s["kl_k3"] - kl_pq) <= 5 * se3
    assert abs(kl_qp - kl_pq) > 100 * max(se1, se3) and 2 * kl_pq > 100 * max(se1, se3)
    # E[w] = sum_v p_v q_v / p_v = 1 under the rollout's own sampling
    assert abs(s["weight_mean"] - 1.0) <= 5 * np.std(np.exp(d)) / math.sqrt(n)


def test_k2_close_to_kl_for_close_policies():
    """For q close to p, E[k2] = KL(p || q) + O(|q - p|^3)."""
    rng = np.random.default_rng(7)
    V = 40
    p = rng.dirichlet(np.ones(V) * 5)
    q = p * np.exp(rng.normal(0, 0.05, V))
    q /= q.sum()
    y = rng.choice(V, size=400_000, p=p)
    s = oracle.mismatch_stats(np.log(q)[y], np.log(p)[y])
    kl = float(np.sum(p * (np.log(p) - np.log(q))))
    assert abs(s["kl_k2"] - kl) <= 0.1 * kl


def _delta_for_deviation(dev):
    """delta with |exp(delta) - 1| = dev (up to rounding), w above 1."""
    return np.log1p(np.asarray(dev, dtype=np.float64))


@pytest.mark.parametrize("devs,median", [([3.0, 1.0, 2.0], 2.0), ([4.0, 1.0, 3.0, 2.0], 2.5), ([5.0], 5.0),
                                          ([1.0, 1.0, 1.0, 10.0], 1.0)])
def test_median_and_peak_of_hand_sorted_deviations(devs, median):
    d = _delta_for_deviation(devs)
    s = oracle.mismatch_stats(d, np.zeros_like(d))
    assert abs(s["deviation_median"] - median) <= 1e-14 * median
    assert abs(s["deviation_max"] - max(devs)) <= 1e-14 * max(devs)
    assert abs(s["deviation_peak_over_median"] - max(devs) / median) <= 1e-13 * max(devs) / median


def test_weight_below_one_counts_its_distance():
    """w = 1/2 is a deviation of 1/2, w = 2 one of 1."""
    s = oracle.mismatch_stats(np.array([-LN2, LN2]), np.zeros(2))
    assert abs(s["deviation_median"] - 0.75) <= 1e-15
    assert abs(s["deviation_max"] - 1.0) <= 1e-15
    assert abs(s["weight_min"] - 0.5) <= 1e-15


def test_zero_median_with_nonzero_peak_is_infinite():
    s = oracle.mismatch_stats(np.array([0.0, 0.0, 0.0, 0.5]), np.zeros(4))
    assert s["deviation_median"] == 0.0 and s["deviation_peak_over_median"] == math.inf


def test_split_telescopes_and_counts_bits():
    rng = np.random.default_rng(3)
    n = 5000
    lr = rng.normal(-2, 1, n).astype(np.float32)
    same = lr.copy()
    same[::7] = np.nextafter(same[::7], np.float32(0))  # a one-ulp kernel mismatch on every 7th token
    same[3] = np.float32(-0.0) if lr[3] == 0 else same[3]
    lp = (same + rng.normal(0, 0.02, n)).astype(np.float32)
    s = oracle.mismatch_stats(lp, lr, same)
    assert s["kernel_nonzero"] == len(range(0, n, 7))
    lag = lp.astype(np.float64) - same.astype(np.float64)
    ker = same.astype(np.float64) - lr.astype(np.float64)
    assert np.allclose(lag + ker, lp.astype(np.float64) - lr.astype(np.float64), rtol=0, atol=1e-15)
    assert 0 < s["kernel_abs_max"] <= 4.8e-7 * np.max(np.abs(lr))  # one ulp of the largest value, at most
    assert s["lag_abs_max"] > 100 * s["kernel_abs_max"]
    # a pure sign-of-zero difference is a bit difference with zero size
    z = oracle.mismatch_stats(np.zeros(1, np.float32), np.array([-0.0], np.float32), np.zeros(1, np.float32))
    assert z["kernel_nonzero"] == 1 and z["kernel_abs_max"] == 0.0


def test_estimators_nonnegative_where_they_must_be():
    rng = np.random.default_rng(4)
    lp = rng.normal(-2, 1, 3000)
    lr = lp + rng.normal(0, 0.3, 3000)
    s = oracle.mismatch_stats(lp, lr, lr)
    assert s["kl_k2"] >= 0 and s["kl_k3"] >= 0 and s["lag_kl_k3"] >= 0 and s["kernel_kl_k3"] == 0


def test_empty_and_no_split():
    e = oracle.mismatch_stats(np.zeros(0), np.zeros(0))
    assert e["n_tok"] == 0 and all(math.isnan(e[k]) for k in oracle.STAT_NAMES if k != "n_tok")
    s = oracle.mismatch_stats(np.array([-1.0]), np.array([-1.5]))
    assert math.isnan(s["lag_abs_mean"]) and math.isnan(s["kernel_nonzero"])
    assert abs(s["kl_k1"] + 0.5) <= 1e-15
