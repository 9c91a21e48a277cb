"""The oracle against hand-derived worked cases (tests/golden/hand_examples.json).

Each case cites the passage whose definition it exercises; expected values
are closed forms written out here with math, independent of the oracle.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle

CASES = {c["id"]: c for c in json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))["cases"]}


def test_every_case_cites_a_passage():
    for c in CASES.values():
        assert "section" in c["cite"] or "definition" in c["cite"] or "as above" in c["cite"]


def test_advantage_two_groups():
    c = CASES["advantage_two_groups"]
    A = oracle.group_advantage(c["rewards"], c["group_offsets"])
    assert np.allclose(A, c["expected"], rtol=0, atol=1e-15)


def test_logprob_tiny_head():
    c = CASES["logprob_tiny_head"]
    lp, lse = oracle.lmhead_logprob(np.array(c["H"]), np.array(c["W"]), np.array(c["tokens"]))
    e = math.e
    want = [1.0 - math.log(2 * e + 1), 2.0 - math.log(1 + 2 * e * e)]
    assert np.allclose(lp, want, rtol=0, atol=1e-15)
    assert np.allclose(lse, [math.log(2 * e + 1), math.log(1 + 2 * e * e)], rtol=0, atol=1e-15)


def test_logprob_uniform_vocab():
    c = CASES["logprob_uniform_vocab"]
    H = np.zeros((3, c["d"]))
    W = np.random.default_rng(0).normal(size=(c["vocab"], c["d"]))
    lp, _ = oracle.lmhead_logprob(H, W, np.array([0, 511, 1023]))
    assert np.all(lp == -10 * math.log(2)) or np.allclose(lp, -10 * math.log(2), rtol=0, atol=1e-15)


def test_loss_one_group_two_responses():
    c = CASES["loss_one_group_two_responses"]
    A = oracle.group_advantage(c["rewards"], c["group_offsets"])
    rl, L, coef = oracle.reinforce_zero_loss(np.array(c["logprob"]), np.array(c["rollout_logprob"]), A,
                                             np.array(c["resp_offsets"]))
    e = math.exp
    l0 = -0.5 * (e(0.5) + 1.0) / 2
    l1 = 0.5 * e(-1.0)
    assert abs(rl[0] - l0) <= 1e-15 and abs(rl[1] - l1) <= 1e-15
    assert abs(L - (l0 + l1) / 2) <= 1e-15
    assert np.allclose(coef, [-e(0.5) / 8, -1 / 8, e(-1.0) / 4], rtol=1e-15, atol=0)


def test_ratio_unclipped():
    c = CASES["ratio_unclipped"]
    r = oracle.importance_ratio(c["logprob"], c["rollout_logprob"])
    assert r[0] == 1.0
    assert r[1] == pytest.approx(math.exp(5.0), rel=1e-15)
    assert r[2] == pytest.approx(math.exp(30.0), rel=1e-15)


def test_mismatch_stats_mixed():
    c = CASES["mismatch_stats_mixed"]
    lr = np.array(c["rollout_logprob"])
    ln2 = math.log(2.0)
    lp = lr + np.array([ln2, 0.0, -ln2, ln2])
    s = oracle.mismatch_stats(lp, lr)
    want = {"kl_k1": -ln2 / 4, "kl_k2": 3 * ln2 * ln2 / 8, "kl_k3": (1.5 - ln2) / 4, "weight_mean": 11 / 8,
            "weight_max": 2.0, "weight_min": 0.5, "deviation_max": 1.0, "deviation_median": 0.75,
            "deviation_peak_over_median": 4 / 3}
    for k, v in want.items():
        assert abs(s[k] - v) <= 1e-15 * max(1.0, abs(v)), k
