"""Oracle: train/inference mismatch diagnostics over sampled-token logprobs
(float64, CPU).

TEST INFRASTRUCTURE -- see the package docstring for who may use it.

Sources (web pages, cited by title and section):

* "vLLM says aligned kernels make asynchronous RL stable at lag 64", section
  "Asynchronous training has two different gaps": the learner/rollout logprob difference splits
  into weight lag (different policy versions, same computation) and kernel
  mismatch (same weights and tokens, different values from the two engines);
  the importance-weight deviation is reported as its peak over its median
  (1.50x with aligned kernels against 442.54x with standard ones).
* The same page, section "REINFORCE Zero removes the mismatch first": the
  importance weight of a token is the learner's probability over the
  rollout's recorded probability, exp(lp - lp_rollout), unclipped.
* "vLLM Train-Inference Consistency Release Notes", section "The Technical
  Challenge: Train-Inference Mismatch": the train-inference KL divergence is
  the mismatch measure tracked over training.

The pages name these statistics but give no formula. Readings taken here:

* delta_t = lp_t - lp_rollout_t (learner minus rollout), w_t = exp(delta_t).
* KL: the rollout-to-learner divergence KL(pi_rollout || pi_learner),
  estimated from the sampled tokens (drawn from the rollout policy) with the
  three standard per-sample estimators of J. Schulman's note "Approximating
  KL Divergence" (2020): k1 = -delta, k2 = delta^2 / 2,
  k3 = (w - 1) - delta = expm1(delta) - delta, each averaged over tokens.
  k1 and k3 are unbiased; k3 is never negative.
* Deviation of the weight: dev_t = |w_t - 1|. Peak = max dev, median = the
  median of dev (the mean of the two middle values for an even count); the
  reported ratio is peak / median, 1 when both are 0, +inf when only the
  median is 0.
* Split (needs lp_same: the learner's computation at the rollout's weights):
  lag_t = lp_t - lp_same_t, kernel_t = lp_same_t - lp_rollout_t, so
  lag_t + kernel_t = delta_t. Per part: mean |.|, max |.| and the k3
  estimator of the part; kernel_nonzero counts the tokens whose float32
  lp_same and lp_rollout differ in any bit (the pages' "bitwise identical").
  Without lp_same these fields are NaN.
* Empty input: n_tok = 0 and every other field NaN.

Pins (tests/test_oracle_diagnostics.py, tests/test_golden.py): closed forms
(w = 2 exactly for delta = ln 2, constant shifts), a hand-worked mixed case,
Monte-Carlo unbiasedness of k1 and k3 against the exact KL of two known
categorical distributions (fixes the direction and sign), k2 ~ KL for close
distributions, medians of hand-sorted arrays, the telescoping split, and
bit-level counting of the kernel part.
"""

import math

import numpy as np

STAT_NAMES = (
    "n_tok",
    "kl_k1",
    "kl_k2",
    "kl_k3",
    "weight_mean",
    "weight_max",
    "weight_min",
    "deviation_max",
    "deviation_median",
    "deviation_peak_over_median",
    "lag_abs_mean",
    "lag_abs_max",
    "lag_kl_k3",
    "kernel_abs_mean",
    "kernel_abs_max",
    "kernel_kl_k3",
    "kernel_nonzero",
)


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _median(v):
    """Median by sorting: the middle value, or the mean of the two middle
    values for an even count."""
    s = np.sort(v)
    n = s.size
    if n % 2 == 1:
        return float(s[n // 2])
    return float((s[n // 2 - 1] + s[n // 2]) / 2.0)


def _k3(delta):
    return np.expm1(delta) - delta


def mismatch_stats(lp, lp_rollout, lp_same=None):
    """Mismatch statistics of one batch of sampled tokens, as a dict keyed
    by STAT_NAMES. lp, lp_rollout and lp_same are per-token logprobs; float32
    arrays keep their bits for kernel_nonzero, every other field is computed
    in float64 from their exact values."""
    lp32 = np.asarray(lp)
    lr32 = np.asarray(lp_rollout)
    n = int(lp32.size)
    out = {k: math.nan for k in STAT_NAMES}
    out["n_tok"] = float(n)
    if n == 0:
        return out
    delta = _f64(lp32) - _f64(lr32)
    w = np.exp(delta)
    dev = np.abs(np.expm1(delta))
    out["kl_k1"] = float(np.mean(-delta))
    out["kl_k2"] = float(np.mean(delta * delta / 2.0))
    out["kl_k3"] = float(np.mean(_k3(delta)))
    out["weight_mean"] = float(np.mean(w))
    out["weight_max"] = float(np.max(w))
    out["weight_min"] = float(np.min(w))
    peak = float(np.max(dev))
    med = _median(dev)
    out["deviation_max"] = peak
    out["deviation_median"] = med
    if med > 0.0:
        out["deviation_peak_over_median"] = peak / med
    else:
        out["deviation_peak_over_median"] = 1.0 if peak == 0.0 else math.inf
    if lp_same is not None:
        ls32 = np.asarray(lp_same)
        lag = _f64(lp32) - _f64(ls32)
        ker = _f64(ls32) - _f64(lr32)
        out["lag_abs_mean"] = float(np.mean(np.abs(lag)))
        out["lag_abs_max"] = float(np.max(np.abs(lag)))
        out["lag_kl_k3"] = float(np.mean(_k3(lag)))
        out["kernel_abs_mean"] = float(np.mean(np.abs(ker)))
        out["kernel_abs_max"] = float(np.max(np.abs(ker)))
        out["kernel_kl_k3"] = float(np.mean(_k3(ker)))
        a = np.ascontiguousarray(ls32, dtype=np.float32).view(np.uint32)
        b = np.ascontiguousarray(lr32, dtype=np.float32).view(np.uint32)
        out["kernel_nonzero"] = float(np.count_nonzero(a != b))
    return out
