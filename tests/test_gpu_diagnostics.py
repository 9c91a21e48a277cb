"""GPU parity of itl_mismatch_stats against the float64 oracle.

The GPU computes every per-token term in fp64 from the fp32 inputs (as the
oracle does) and sums in a different, fixed order: sums must agree to 1e-12
relative to the sum of the terms' magnitudes; maxima, minima and the median
are single per-token values and agree to 1e-14 relative; the bit-difference
count is exact. Cases span one token, odd and even counts, several 2048-token
workgroups with a ragged tail, the qwen3-4b head's token count with its lag
noise recipe, middle values far apart and tied values, zero lag (every key
equal) and the empty batch.
"""

import math

import numpy as np
import pytest

from helpers import say

pytestmark = pytest.mark.gpu

SUM_TOL = 1e-12
VAL_TOL = 1e-14


def _itl():
    import invariant_token_logprobs_lm_amd as itl

    return itl


def _scales(lp, lr, ls):
    d = lp.astype(np.float64) - lr.astype(np.float64)
    sc = {"kl_k1": np.mean(np.abs(d)), "kl_k2": np.mean(d * d / 2), "kl_k3": np.mean(np.abs(np.expm1(d) - d)),
          "weight_mean": np.mean(np.exp(d))}
    if ls is not None:
        lag = lp.astype(np.float64) - ls.astype(np.float64)
        ker = ls.astype(np.float64) - lr.astype(np.float64)
        sc.update({"lag_abs_mean": np.mean(np.abs(lag)), "lag_kl_k3": np.mean(np.abs(np.expm1(lag) - lag)),
                   "kernel_abs_mean": np.mean(np.abs(ker)), "kernel_kl_k3": np.mean(np.abs(np.expm1(ker) - ker))})
    return sc


def _compare(got, want, scales, label):
    worst = 0.0
    for k, w in want.items():
        g = got[k]
        if isinstance(w, float) and math.isnan(w):
            assert math.isnan(g), (label, k, g)
            continue
        if k in ("n_tok", "kernel_nonzero"):
            assert g == w, (label, k, g, w)
            continue
        if math.isinf(w) or w == 0.0 and k not in scales:
            assert g == w, (label, k, g, w)
            continue
        if k in scales:
            tol = SUM_TOL * max(scales[k], 1e-300)
        else:
            tol = VAL_TOL * abs(w)
        err = abs(g - w)
        worst = max(worst, err / max(abs(w), 1e-300))
        assert err <= tol, (label, k, g, w, err, tol)
    say(f"[diagnostics {label}] n={int(want['n_tok'])}: worst rel {worst:.2e}, "
        f"peak/median {got['deviation_peak_over_median']:.4g}, k3 {got['kl_k3']:.4g}")


def _run(lp, lr, ls, cuda, label):
    import torch
    import oracle

    itl = _itl()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(cuda)
    st = itl.mismatch_stats(t(lp), t(lr), None if ls is None else t(ls))
    got = itl.stats_dict(st)
    want = oracle.mismatch_stats(lp, lr, ls)
    _compare(got, want, _scales(lp, lr, ls), label)
    st2 = itl.mismatch_stats(t(lp), t(lr), None if ls is None else t(ls))
    torch.cuda.synchronize()
    assert torch.equal(st.view(torch.int64), st2.view(torch.int64))  # run-to-run bits
    return got


def _lagged(n, seed, heavy=0.01):
    """Rollout record = learner + N(0, 0.05), plus N(0, 1) on a Bernoulli(heavy)
    subset (the qwen3-4b workload's lag-noise recipe)."""
    rng = np.random.default_rng(seed)
    lp = -np.abs(rng.standard_normal(n) * 2).astype(np.float32)
    noise = rng.normal(0, 0.05, n) + (rng.random(n) < heavy) * rng.normal(0, 1, n)
    lr = (lp + noise).astype(np.float32)
    same = lr.copy()
    flip = rng.random(n) < 0.1
    same[flip] = np.nextafter(same[flip], np.float32(0))
    return lp, lr, same


@pytest.mark.parametrize("n", [1, 2, 7, 2048, 2049, 100_003])
def test_parity_random(cuda, n):
    lp, lr, same = _lagged(n, seed=n)
    _run(lp, lr, same, cuda, f"lagged+split n={n}")
    _run(lp, lr, None, cuda, f"lagged n={n}")


def test_median_between_far_apart_values(cuda):
    """The two middle deviations lie in different 16-bit key prefixes (two
    clusters), and many deviations tie: the median is still exact."""
    rng = np.random.default_rng(11)
    n = 4000
    lp = -np.abs(rng.standard_normal(n)).astype(np.float32)
    shift = np.where(np.arange(n) < n // 2, 0.25, 1.5).astype(np.float32)  # half small, half large deviations
    lr = (lp + shift).astype(np.float32)
    rng.shuffle(lr)  # also breaks the pairing: deviations spread over many values
    lr[: n // 4] = lp[: n // 4] + np.float32(0.25)  # a block of tied values
    _run(lp, lr, None, cuda, "two clusters with ties")
    lr2 = lp + np.where(np.arange(n) % 2 == 0, np.float32(1e-3), np.float32(3.0)).astype(np.float32)
    got = _run(lp, lr2.astype(np.float32), None, cuda, "two-valued")
    assert got["deviation_median"] > 0


def test_zero_lag_is_exact(cuda):
    lp = -np.abs(np.random.default_rng(2).standard_normal(5000)).astype(np.float32)
    got = _run(lp, lp.copy(), lp.copy(), cuda, "zero lag")
    for k in ("kl_k1", "kl_k2", "kl_k3", "deviation_max", "deviation_median", "kernel_abs_max", "kernel_nonzero"):
        assert got[k] == 0.0, k
    assert got["weight_min"] == 1.0 and got["weight_max"] == 1.0 and got["deviation_peak_over_median"] == 1.0


def test_empty_batch(cuda):
    import torch

    itl = _itl()
    e = torch.empty(0, dtype=torch.float32, device=cuda)
    got = itl.stats_dict(itl.mismatch_stats(e, e, e))
    assert got["n_tok"] == 0 and all(math.isnan(got[k]) for k in itl.STAT_FIELDS if k != "n_tok")


def test_full_size_head_split(cuda):
    """The qwen3-4b head at full token count: learner logprobs from the
    library's own kernel, a rollout record with the workload's lag noise, and
    a rollout that is the same kernel at the same weights (kernel part exactly
    zero)."""
    import torch
    from synth import WORKLOADS, draw_head, draw_layout, sample_tokens

    itl = _itl()
    wl = WORKLOADS["qwen3-4b-head"]
    lay = draw_layout(wl)
    H, W = draw_head(wl, lay.n_tok, device=cuda)
    y = sample_tokens(H, W, wl)
    lp, _ = itl.lmhead_logprob(H, W, y)
    lr = lp + torch.from_numpy(lay.lag_noise).to(cuda)
    lp_h, lr_h = lp.cpu().numpy(), lr.cpu().numpy()
    # aligned rollout: the learner's kernel at the rollout's weights
    # reproduces the rollout record bit for bit, so the whole gap is weight lag
    got = _run(lp_h, lr_h, lr_h.copy(), cuda, "qwen3-4b-head, aligned")
    assert got["kernel_nonzero"] == 0.0 and got["kernel_abs_max"] == 0.0
    assert got["lag_abs_max"] > 0
    # the opposite split: same weights as the learner, the gap all kernel
    got = _run(lp_h, lr_h, lp_h.copy(), cuda, "qwen3-4b-head, gap all kernel")
    assert got["lag_abs_max"] == 0.0 and got["kernel_nonzero"] == float(np.count_nonzero(
        lp_h.view(np.uint32) != lr_h.view(np.uint32)))
