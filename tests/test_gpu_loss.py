"""GPU parity of itl_group_advantage and itl_reinforce_zero_loss.

Bar: advantages within 1e-6 absolute (rewards are O(1)); per-response loss,
loss and coef within 1e-3 relative of the float64 oracle on the same inputs;
exact identities at zero lag; bitwise invariance of a group's advantages and
a response's loss under reordering of the batch.
"""

import numpy as np
import pytest

from helpers import rel_err, same_bits, say

pytestmark = pytest.mark.gpu

TOL_REL = 1e-3


def _itl():
    import invariant_token_logprobs_lm_amd as itl

    return itl


def _gpu_loss(lp, lpr, A, off, cuda):
    import torch

    itl = _itl()
    t = lambda a, dt: torch.as_tensor(np.ascontiguousarray(a), dtype=dt, device=cuda)
    return itl.reinforce_zero_loss(t(lp, torch.float32), t(lpr, torch.float32), t(A, torch.float32),
                                   t(off, torch.int64))


def _check_loss(lp, lpr, A, off, cuda, label):
    import oracle

    rl, L, c = _gpu_loss(lp, lpr, A, off, cuda)
    rl_o, L_o, c_o = oracle.reinforce_zero_loss(lp.astype(np.float64), lpr.astype(np.float64),
                                                A.astype(np.float64), off)
    e1 = float(rel_err(rl.cpu().numpy(), rl_o).max())
    e2 = float(rel_err([L.item()], [L_o]).max())
    e3 = float(rel_err(c.cpu().numpy(), c_o).max()) if c_o.size else 0.0
    say(f"[loss {label}] N={A.size} n_tok={lp.size}: rel resp_loss={e1:.2e} loss={e2:.2e} coef={e3:.2e}")
    assert e1 <= TOL_REL and e3 <= TOL_REL
    # loss is a mean of signed terms: relative error is measured against the
    # sum of magnitudes when the mean nearly cancels
    scale = max(abs(L_o), float(np.abs(rl_o).mean()))
    assert abs(L.item() - L_o) <= TOL_REL * scale
    return rl, L, c


@pytest.mark.parametrize("sizes", [[8] * 8, [16] * 4, [1, 3, 64, 65, 100, 200, 2], [4] * 1000])
def test_group_advantage_parity(cuda, sizes):
    import torch
    import oracle

    itl = _itl()
    rng = np.random.default_rng(len(sizes))
    goff = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    r = rng.random(goff[-1]).astype(np.float32)
    A = itl.group_advantage(torch.from_numpy(r).to(cuda), torch.from_numpy(goff).to(cuda))
    A_o = oracle.group_advantage(r, goff)
    err = float(np.max(np.abs(A.cpu().numpy() - A_o)))
    say(f"[advantage] groups={len(sizes)} max|dA|={err:.2e}")
    assert err <= 1e-6


def test_group_advantage_binary_rewards_cancel_exactly(cuda):
    import torch

    itl = _itl()
    rng = np.random.default_rng(0)
    gs, G = 8, 64
    r = (rng.random(G * gs) < 0.3).astype(np.float32)
    goff = (np.arange(G + 1) * gs).astype(np.int32)
    A = itl.group_advantage(torch.from_numpy(r).to(cuda), torch.from_numpy(goff).to(cuda)).cpu().numpy()
    for g in range(G):
        assert float(np.sum(A[g * gs:(g + 1) * gs].astype(np.float64))) == 0.0


def test_group_advantage_position_invariance(cuda):
    import torch

    itl = _itl()
    rng = np.random.default_rng(1)
    sizes = [5, 8, 77, 3]
    goff = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    r = rng.random(goff[-1]).astype(np.float32)
    A = itl.group_advantage(torch.from_numpy(r).to(cuda), torch.from_numpy(goff).to(cuda))
    perm = [2, 0, 3, 1]
    r2 = np.concatenate([r[goff[g]:goff[g + 1]] for g in perm])
    goff2 = np.concatenate([[0], np.cumsum([sizes[g] for g in perm])]).astype(np.int32)
    A2 = itl.group_advantage(torch.from_numpy(r2).to(cuda), torch.from_numpy(goff2).to(cuda))
    for k, g in enumerate(perm):
        assert same_bits(A[goff[g]:goff[g + 1]], A2[goff2[k]:goff2[k + 1]])


def test_loss_tiny_end_to_end(cuda):
    """Tiny workload: GPU logprob -> GPU advantage -> GPU loss, against the
    oracle's own chain from the same head, tokens, rollout record and rewards."""
    import torch
    import oracle
    from synth import WORKLOADS, draw_head, draw_layout, sample_tokens

    itl = _itl()
    wl = WORKLOADS["tiny"]
    lay = draw_layout(wl)
    H, W = draw_head(wl, lay.n_tok, device="cpu")
    y = sample_tokens(H, W, wl)
    lp_o, _ = oracle.lmhead_logprob(H.numpy(), W.numpy(), y.numpy())
    lpr = (lp_o + lay.lag_noise).astype(np.float32)  # the rollout's record
    A_o = oracle.group_advantage(lay.rewards, lay.group_offsets)
    rl_o, L_o, c_o = oracle.reinforce_zero_loss(lp_o, lpr.astype(np.float64), A_o, lay.resp_offsets)

    lp, _ = itl.lmhead_logprob(H.to(cuda), W.to(cuda), y.to(cuda))
    A = itl.group_advantage(torch.from_numpy(lay.rewards).to(cuda), torch.from_numpy(lay.group_offsets).to(cuda))
    rl, L, c = itl.reinforce_zero_loss(lp, torch.from_numpy(lpr).to(cuda), A,
                                       torch.from_numpy(lay.resp_offsets).to(cuda))
    e1 = float(rel_err(rl.cpu().numpy(), rl_o).max())
    e3 = float(rel_err(c.cpu().numpy(), c_o).max())
    scale = max(abs(L_o), float(np.abs(rl_o).mean()))
    say(f"[tiny e2e] rel resp_loss={e1:.2e} coef={e3:.2e} |dL|/scale={abs(L.item() - L_o) / scale:.2e}")
    assert e1 <= TOL_REL and e3 <= TOL_REL and abs(L.item() - L_o) <= TOL_REL * scale


@pytest.mark.parametrize("key", ["qwen2.5-1.5b-head", "qwen3-4b-head", "large-moe-head"])
def test_loss_full_size_layouts(cuda, key):
    """Full-size response layouts with synthetic learner logprobs."""
    from synth import WORKLOADS, draw_layout, synthetic_logprobs
    import oracle

    wl = WORKLOADS[key]
    lay = draw_layout(wl)
    lp = synthetic_logprobs(lay.n_tok, seed=wl.index)
    lpr = (lp + lay.lag_noise).astype(np.float32)
    A = oracle.group_advantage(lay.rewards, lay.group_offsets).astype(np.float32)
    _check_loss(lp, lpr, A, lay.resp_offsets, cuda, key)


def test_loss_many_short_responses(cuda):
    rng = np.random.default_rng(5)
    N = 20000
    T = rng.integers(1, 17, N)
    off = np.concatenate([[0], np.cumsum(T)]).astype(np.int64)
    lp = -np.abs(rng.normal(5, 2, off[-1])).astype(np.float32)
    lpr = (lp + rng.normal(0, 0.1, off[-1])).astype(np.float32)
    A = rng.normal(0, 1, N).astype(np.float32)
    _check_loss(lp, lpr, A, off, cuda, "many short")


def test_zero_lag_identities(cuda):
    """lp_rollout == lp bitwise: ratio = 1 exactly, resp_loss = -A exactly,
    coef = the plain REINFORCE coefficient, loss = 0 for binary rewards in
    power-of-two groups."""
    import torch

    itl = _itl()
    rng = np.random.default_rng(9)
    G, gs = 4, 8
    T = rng.integers(3, 3000, G * gs)
    off = np.concatenate([[0], np.cumsum(T)]).astype(np.int64)
    lp = -np.abs(rng.normal(4, 2, off[-1])).astype(np.float32)
    r = (rng.random(G * gs) < 0.5).astype(np.float32)
    goff = (np.arange(G + 1) * gs).astype(np.int32)
    A = itl.group_advantage(torch.from_numpy(r).to(cuda), torch.from_numpy(goff).to(cuda))
    lp_t = torch.from_numpy(lp).to(cuda)
    rl, L, c = itl.reinforce_zero_loss(lp_t, lp_t.clone(), A, torch.from_numpy(off).to(cuda))
    assert torch.equal(rl, -A)
    assert L.item() == 0.0
    Ah = A.cpu().numpy().astype(np.float64)
    want = np.repeat((-Ah / (G * gs * T)).astype(np.float32), T)
    assert np.array_equal(c.cpu().numpy(), want)


def test_ratio_is_not_clipped(cuda):
    lp = np.array([-1.0, -1.0, -1.0, -1.0], np.float32)
    lpr = np.array([-51.0, -1.0, -200.0, -1.0], np.float32)
    A = np.array([1.0, -1.0], np.float32)
    off = np.array([0, 2, 4], np.int64)
    rl, _, c = _gpu_loss(lp, lpr, A, off, cuda)
    rl = rl.cpu().numpy()
    assert abs(rl[0] - (-(np.exp(50.0) + 1.0) / 2)) <= 1e-5 * np.exp(50.0)
    assert np.isinf(rl[1])  # exp(199) overflows fp32: +inf, never clamped


def test_response_loss_batch_invariance(cuda):
    import torch

    rng = np.random.default_rng(12)
    N = 40
    T = rng.integers(1, 5000, N)
    off = np.concatenate([[0], np.cumsum(T)]).astype(np.int64)
    lp = -np.abs(rng.normal(6, 2, off[-1])).astype(np.float32)
    lpr = (lp + rng.normal(0, 0.05, off[-1])).astype(np.float32)
    A = rng.normal(0, 1, N).astype(np.float32)
    rl, _, _ = _gpu_loss(lp, lpr, A, off, cuda)
    perm = rng.permutation(N)[:17]
    idx = np.concatenate([np.arange(off[i], off[i + 1]) for i in perm])
    off2 = np.concatenate([[0], np.cumsum(T[perm])]).astype(np.int64)
    rl2, _, _ = _gpu_loss(lp[idx], lpr[idx], A[perm], off2, cuda)
    assert same_bits(rl[torch.from_numpy(perm).to(cuda)], rl2)


def test_response_loss_across_the_short_long_boundary(cuda):
    """Responses just below, at and above the lengths where the sum changes
    tree (eight lanes / one wavefront / one workgroup), mixed with others: parity with the oracle, and each response's loss has the same
    bits alone, in the batch, and in a permuted sub-batch."""
    import re
    import torch

    itl = _itl()
    short = int(re.search(r"short_response=(\d+)", itl.build_info()).group(1))
    tiny = int(re.search(r"tiny_response=(\d+)", itl.build_info()).group(1))
    lens = [1, tiny - 1, tiny, tiny + 1, 63, 64, 65, short - 1, short, short + 1, 1000, 2 * short + 3, 7]
    rng = np.random.default_rng(21)
    T = np.array(lens * 3)
    N = T.size
    off = np.concatenate([[0], np.cumsum(T)]).astype(np.int64)
    lp = -np.abs(rng.normal(6, 2, off[-1])).astype(np.float32)
    lpr = (lp + rng.normal(0, 0.05, off[-1])).astype(np.float32)
    A = rng.normal(0, 1, N).astype(np.float32)
    rl, _, c = _check_loss(lp, lpr, A, off, cuda, "short/long boundary")
    for i in range(len(lens)):
        rl1, _, _ = _gpu_loss(lp[off[i]:off[i + 1]], lpr[off[i]:off[i + 1]], A[i:i + 1],
                              np.array([0, T[i]], dtype=np.int64), cuda)
        assert same_bits(rl1, rl[i:i + 1]), lens[i]
    perm = rng.permutation(N)[:11]
    idx = np.concatenate([np.arange(off[i], off[i + 1]) for i in perm])
    off2 = np.concatenate([[0], np.cumsum(T[perm])]).astype(np.int64)
    rl2, _, _ = _gpu_loss(lp[idx], lpr[idx], A[perm], off2, cuda)
    assert same_bits(rl[torch.from_numpy(perm).to(cuda)], rl2)


def test_loss_many_responses_mean(cuda):
    """Many responses (the mean's 16-byte passes and its ragged end): parity
    of the loss and run-to-run bit equality."""
    rng = np.random.default_rng(8)
    N = 100003
    T = rng.integers(1, 40, N)
    off = np.concatenate([[0], np.cumsum(T)]).astype(np.int64)
    lp = -np.abs(rng.normal(5, 2, off[-1])).astype(np.float32)
    lpr = (lp + rng.normal(0, 0.1, off[-1])).astype(np.float32)
    A = rng.normal(0, 1, N).astype(np.float32)
    _, L, _ = _check_loss(lp, lpr, A, off, cuda, "many responses")
    _, L2, _ = _gpu_loss(lp, lpr, A, off, cuda)
    assert same_bits(L, L2)
