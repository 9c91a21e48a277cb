"""The seeded input generators: shapes, ranges and the stated distributions."""

import numpy as np
import pytest

from synth import WORKLOADS, draw_layout, invariance_plan, synthetic_logprobs, token_subset


@pytest.mark.parametrize("key", list(WORKLOADS))
def test_layout_shapes_and_ranges(key):
    wl = WORKLOADS[key]
    lay = draw_layout(wl)
    assert lay.n_resp == wl.n_groups * wl.group_size
    assert lay.lengths.min() >= wl.len_lo and lay.lengths.max() <= wl.len_hi
    assert lay.resp_offsets[0] == 0 and np.all(np.diff(lay.resp_offsets) == lay.lengths)
    assert lay.group_offsets.dtype == np.int32 and lay.group_offsets[-1] == lay.n_resp
    assert lay.lag_noise.shape == (lay.n_tok,) and lay.lag_noise.dtype == np.float32
    if wl.reward[0] == "bernoulli":
        assert set(np.unique(lay.rewards)) <= {0.0, 1.0}
    else:
        assert lay.rewards.min() >= 0 and lay.rewards.max() < 1
    # deterministic
    again = draw_layout(wl)
    assert np.array_equal(again.lag_noise, lay.lag_noise) and np.array_equal(again.rewards, lay.rewards)


def test_lag_noise_statistics():
    lay = draw_layout(WORKLOADS["qwen2.5-1.5b-head"])
    x = lay.lag_noise.astype(np.float64)
    assert abs(x.mean()) < 5 * 0.02 / np.sqrt(x.size)
    assert abs(x.std() - 0.02) < 0.02 * 0.01
    lay3 = draw_layout(WORKLOADS["qwen3-4b-head"])
    x3 = lay3.lag_noise.astype(np.float64)
    frac_tail = np.mean(np.abs(x3) > 0.4)  # 8 sigma of the base noise
    assert 0.006 < frac_tail < 0.012
    # variance = base^2 + 1% * 1^2
    assert abs(x3.var() - (0.05**2 + 0.01)) < 0.1 * (0.05**2 + 0.01)


def test_reduced_instance_and_plan():
    wl = WORKLOADS["large-moe-head"]
    lay = draw_layout(wl, n_groups=1, group_size=16, len_lo=8, len_hi=64)
    assert lay.n_resp == 16 and 16 * 8 <= lay.n_tok <= 16 * 64
    batches, prefill = invariance_plan(draw_layout(WORKLOADS["invariance-stress"]))
    assert len(batches) == 10
    for b in batches:
        assert 1 <= b.size <= 64 and np.unique(b).size == b.size
    assert np.all(prefill >= 1)


def test_subset_and_synthetic_logprobs():
    s = token_subset(1000, 50, 1)
    assert s.size == 50 and np.all(np.diff(s) > 0) and s.max() < 1000
    lp = synthetic_logprobs(1000, 2)
    assert np.all(lp <= 0)


def test_sampler_draws_from_softmax():
    torch = pytest.importorskip("torch")
    from synth import sample_tokens

    wl = WORKLOADS["tiny"]
    d, V, n = 4, 6, 60000
    g = torch.Generator().manual_seed(0)
    H = torch.randn(1, d, generator=g).repeat(n, 1)
    W = torch.randn(V, d, generator=g)
    y = sample_tokens(H, W, wl, chunk_rows=8192).numpy()
    z = (H[0].double() @ W.double().T).numpy()
    p = np.exp(z - z.max())
    p /= p.sum()
    counts = np.bincount(y, minlength=V)
    chi2 = float(((counts - n * p) ** 2 / (n * p)).sum())
    # 5 degrees of freedom: P(chi2 > 25) < 2e-4
    assert chi2 < 25.0
