"""Pins for the oracle's group advantage, ratio, loss and gradient.

Checked against closed forms, exact zero sums, the zero-lag reduction to
plain REINFORCE, central finite differences of the whole loss in float64,
and torch float64 autograd.
"""

import math

import numpy as np
import pytest

import oracle


def test_advantage_hand_example():
    A = oracle.group_advantage([1, 0, 0, 1, 1, 0.25, 0.75], [0, 5, 7])
    assert np.allclose(A, [0.4, -0.6, -0.6, 0.4, 0.4, -0.25, 0.25], atol=1e-15, rtol=0)


@pytest.mark.parametrize("gs", [4, 8, 16])
def test_advantages_sum_to_exactly_zero_for_binary_rewards(gs):
    rng = np.random.default_rng(gs)
    G = 50
    r = (rng.random(G * gs) < 0.4).astype(np.float64)
    A = oracle.group_advantage(r, np.arange(G + 1) * gs)
    for g in range(G):
        assert math.fsum(A[g * gs:(g + 1) * gs]) == 0.0


def test_advantages_sum_to_zero_within_rounding_for_uniform_rewards():
    rng = np.random.default_rng(1)
    gs, G = 8, 100
    r = rng.random(G * gs)
    A = oracle.group_advantage(r, np.arange(G + 1) * gs)
    for g in range(G):
        assert abs(math.fsum(A[g * gs:(g + 1) * gs])) <= 4 * gs * 2.0**-52


def test_equal_rewards_and_singletons_give_zero_advantage():
    A = oracle.group_advantage([0.3] * 6 + [0.9], [0, 6, 7])
    assert np.all(A == 0.0)


def test_advantage_rejects_empty_groups():
    with pytest.raises(ValueError):
        oracle.group_advantage([1.0, 2.0], [0, 0, 2])


def test_ratio_is_exactly_one_at_zero_lag_and_never_clipped():
    lp = -np.abs(np.random.default_rng(2).normal(5, 3, 1000))
    assert np.all(oracle.importance_ratio(lp, lp.copy()) == 1.0)
    r = oracle.importance_ratio(np.array([-1.0, -1.0]), np.array([-51.0, -800.0]))
    assert r[0] == math.exp(50.0)
    assert r[1] == math.inf


def _layout(rng, G, gs, lo, hi):
    lengths = rng.integers(lo, hi, G * gs, endpoint=True)
    off = np.concatenate([[0], np.cumsum(lengths)])
    return lengths, off, np.arange(G + 1) * gs


def test_zero_lag_loss_is_minus_advantage_and_plain_reinforce():
    rng = np.random.default_rng(4)
    lengths, off, goff = _layout(rng, 3, 8, 5, 40)
    r = (rng.random(24) < 0.5).astype(np.float64)
    A = oracle.group_advantage(r, goff)
    lp = -np.abs(rng.normal(3, 1, off[-1]))
    resp_loss, L, coef = oracle.reinforce_zero_loss(lp, lp.copy(), A, off)
    assert np.all(resp_loss == -A)
    assert L == 0.0  # binary rewards, power-of-two groups: advantages cancel exactly
    # plain REINFORCE: J = -(1/N) sum_i (A_i/T_i) sum_t lp_t, dJ/dlp_t = -A_i/(N T_i)
    N = 24
    for i in range(N):
        assert np.all(coef[off[i]:off[i + 1]] == -A[i] / (N * lengths[i]))


def test_loss_hand_example():
    # two responses in one group, rewards 1 and 0 -> A = +0.5, -0.5
    A = oracle.group_advantage([1.0, 0.0], [0, 2])
    lp = np.array([-1.0, -2.0, -3.0])
    lpr = np.array([-1.5, -2.0, -2.0])
    off = np.array([0, 2, 3])
    resp_loss, L, coef = oracle.reinforce_zero_loss(lp, lpr, A, off)
    e = math.exp
    assert abs(resp_loss[0] - (-0.5 * (e(0.5) + 1.0) / 2)) <= 1e-15
    assert abs(resp_loss[1] - (0.5 * e(-1.0))) <= 1e-15
    assert abs(L - (resp_loss[0] + resp_loss[1]) / 2) <= 1e-15
    assert np.allclose(coef, [-e(0.5) * 0.5 / 4, -0.5 / 4, e(-1.0) * 0.5 / 2], rtol=1e-15, atol=0)


def test_per_response_loss_depends_on_its_response_only():
    rng = np.random.default_rng(8)
    lengths, off, goff = _layout(rng, 2, 4, 3, 9)
    lp = -np.abs(rng.normal(2, 1, off[-1]))
    lpr = lp + rng.normal(0, 0.1, off[-1])
    A = rng.normal(0, 1, 8)
    base, _, _ = oracle.reinforce_zero_loss(lp, lpr, A, off)
    perm = rng.permutation(8)
    seg = [np.arange(off[i], off[i + 1]) for i in perm]
    idx = np.concatenate(seg)
    off2 = np.concatenate([[0], np.cumsum(lengths[perm])])
    got, _, _ = oracle.reinforce_zero_loss(lp[idx], lpr[idx], A[perm], off2)
    assert np.all(got == base[perm])


def _tiny_problem(rng, n_groups=2, gs=2, lo=2, hi=4, d=6, V=11, lag=0.3):
    lengths, off, goff = _layout(rng, n_groups, gs, lo, hi)
    n = int(off[-1])
    H = rng.normal(0, 1, (n, d))
    W = rng.normal(0, 0.7, (V, d))
    y = rng.integers(0, V, n)
    lp, _ = oracle.lmhead_logprob(H, W, y)
    lpr = lp + rng.normal(0, lag, n)
    r = rng.random(n_groups * gs)
    A = oracle.group_advantage(r, goff)
    return H, W, y, lpr, A, off


@pytest.mark.parametrize("lag", [0.0, 0.3])
def test_gradient_matches_central_finite_differences(lag):
    rng = np.random.default_rng(21)
    H, W, y, lpr, A, off = _tiny_problem(rng, lag=lag)
    lp, _ = oracle.lmhead_logprob(H, W, y)
    if lag == 0.0:
        lpr = lp.copy()
    _, _, coef = oracle.reinforce_zero_loss(lp, lpr, A, off)
    dH, dW = oracle.reinforce_zero_backward(H, W, y, coef, vocab_chunk=4)
    h = 1e-6

    def L(Hx, Wx):
        return oracle.reinforce_zero_objective(Hx, Wx, y, lpr, A, off)

    for (t, k) in [(0, 0), (1, 3), (H.shape[0] - 1, 5)]:
        Hp, Hm = H.copy(), H.copy()
        Hp[t, k] += h
        Hm[t, k] -= h
        fd = (L(Hp, W) - L(Hm, W)) / (2 * h)
        assert abs(fd - dH[t, k]) <= 1e-7 * max(1e-3, abs(dH).max())
    for (v, k) in [(0, 0), (int(y[0]), 2), (W.shape[0] - 1, 5)]:
        Wp, Wm = W.copy(), W.copy()
        Wp[v, k] += h
        Wm[v, k] -= h
        fd = (L(H, Wp) - L(H, Wm)) / (2 * h)
        assert abs(fd - dW[v, k]) <= 1e-7 * max(1e-3, abs(dW).max())


def test_zero_lag_gradient_equals_plain_reinforce_gradient():
    # At zero lag the REINFORCE Zero gradient is that of
    # J = -(1/N) sum_i (A_i/T_i) sum_t lp_t ; check dH against FD of J.
    rng = np.random.default_rng(31)
    H, W, y, _, A, off = _tiny_problem(rng)
    lp, _ = oracle.lmhead_logprob(H, W, y)
    _, _, coef = oracle.reinforce_zero_loss(lp, lp.copy(), A, off)
    dH, _ = oracle.reinforce_zero_backward(H, W, y, coef)
    N = A.size
    T = np.diff(off)
    w_tok = np.repeat(-A / (N * T), T)

    def J(Hx):
        return float(np.dot(w_tok, oracle.lmhead_logprob(Hx, W, y)[0]))

    h = 1e-6
    for (t, k) in [(0, 1), (2, 4)]:
        Hp, Hm = H.copy(), H.copy()
        Hp[t, k] += h
        Hm[t, k] -= h
        assert abs((J(Hp) - J(Hm)) / (2 * h) - dH[t, k]) <= 1e-7 * max(1e-3, abs(dH).max())


def test_gradient_matches_torch_float64_autograd():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(41)
    H, W, y, lpr, A, off = _tiny_problem(rng, n_groups=2, gs=3, lo=3, hi=7, d=16, V=40)
    lp, _ = oracle.lmhead_logprob(H, W, y)
    _, L, coef = oracle.reinforce_zero_loss(lp, lpr, A, off)
    dH, dW = oracle.reinforce_zero_backward(H, W, y, coef)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    lpt = torch.log_softmax(Ht @ Wt.T, dim=1)[torch.arange(len(y)), torch.tensor(y)]
    ratio = torch.exp(lpt - torch.tensor(lpr))
    terms = []
    for i in range(A.size):
        terms.append(-A[i] * ratio[off[i]:off[i + 1]].mean())
    Lt = torch.stack(terms).mean()
    Lt.backward()
    assert abs(Lt.item() - L) <= 1e-14
    assert np.max(np.abs(Ht.grad.numpy() - dH)) <= 1e-13
    assert np.max(np.abs(Wt.grad.numpy() - dW)) <= 1e-13


def test_dW_columns_sum_to_zero_over_vocab():
    rng = np.random.default_rng(51)
    H, W, y, lpr, A, off = _tiny_problem(rng, d=12, V=300)
    lp, _ = oracle.lmhead_logprob(H, W, y)
    _, _, coef = oracle.reinforce_zero_loss(lp, lpr, A, off)
    _, dW = oracle.reinforce_zero_backward(H, W, y, coef)
    assert np.max(np.abs(dW.sum(axis=0))) <= 1e-13 * max(1e-12, np.abs(dW).max()) * 300


@pytest.mark.parametrize("w_scale", [1.0, 5000.0])
def test_gradient_rows_match_full_gradient(w_scale):
    """The subset evaluator agrees with the full gradient (itself pinned by
    finite differences and float64 autograd above) over a vocabulary of
    several chunks with a ragged last one, including repeated token ids,
    vocabulary rows nobody sampled, and (w_scale 5000) logits spread over
    thousands of units, where exp overflows unless every chunk is shifted by
    the row's true maximum."""
    rng = np.random.default_rng(61)
    H, W, y, lpr, A, off = _tiny_problem(rng, n_groups=2, gs=3, lo=3, hi=7, d=10, V=57)
    W = W * w_scale
    y[:4] = y[0]
    lp, _ = oracle.lmhead_logprob(H, W, y)
    lpr = lp + rng.normal(0, 0.3, lp.size)  # ratios near 1 whatever the scale: every coefficient counts
    _, _, coef = oracle.reinforce_zero_loss(lp, lpr, A, off)
    dH, dW = oracle.reinforce_zero_backward(H, W, y, coef)
    tok = np.array([0, 3, len(y) - 1])
    voc = np.array([int(y[0]), 0, 56, 13])
    dHr, dWr = oracle.reinforce_zero_backward_rows(H, W, y, coef, tok, voc, vocab_chunk=8)
    assert np.max(np.abs(dHr - dH[tok])) <= 1e-13 * np.abs(dH).max()
    assert np.max(np.abs(dWr - dW[voc])) <= 1e-13 * np.abs(dW).max()
