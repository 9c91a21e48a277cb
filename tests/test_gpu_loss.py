"""GPU parity of itl_group_advantage and itl_reinforce_zero_loss.

Bar: advantages within 1e-6 absolute (rewards are O(1)); per-response loss,
loss and coef within 1e-3 relative of the float64 oracle on the same inputs
(an exact zero on one side must be an exact zero on the other); exact
identities at zero lag; bitwise invariance of a group's advantages and a
response's loss under reordering of the batch.
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
    say(f"[loss {label}] N={A.size} n_tok={lp.size}: rel resp_loss={e1:.2e} loss={e2:.2e} "
        f"(|L|={abs(L_o):.3e}, mean|resp_loss|={float(np.abs(rl_o).mean()):.3e}) coef={e3:.2e}")
    assert e1 <= TOL_REL and e2 <= TOL_REL and e3 <= TOL_REL
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
    e2 = float(rel_err([L.item()], [L_o]).max())
    e3 = float(rel_err(c.cpu().numpy(), c_o).max())
    say(f"[tiny e2e] rel resp_loss={e1:.2e} loss={e2:.2e} coef={e3:.2e}")
    assert e1 <= TOL_REL and e2 <= TOL_REL and e3 <= TOL_REL


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


def _loss_constants():
    import re

    info = _itl().build_info()
    get = lambda k: int(re.search(rf"{k}=(\d+)", info).group(1))
    return get("loss_lane_segment"), get("loss_wave_segment"), get("loss_segment_tokens"), get("loss_mean_chunk")


def _alone_batch_permuted(lp, lpr, A, off, rl, idx, cuda, rng):
    """resp_loss of responses idx alone, and of a permuted sub-batch, have the
    bits they have in the full batch."""
    import torch

    T = np.diff(off)
    for i in idx:
        rl1, _, _ = _gpu_loss(lp[off[i]:off[i + 1]], lpr[off[i]:off[i + 1]], A[i:i + 1],
                              np.array([0, T[i]], dtype=np.int64), cuda)
        assert same_bits(rl1, rl[int(i):int(i) + 1]), (int(i), int(T[i]))
    perm = rng.permutation(np.asarray(idx))
    tok = np.concatenate([np.arange(off[i], off[i + 1]) for i in perm])
    off2 = np.concatenate([[0], np.cumsum(T[perm])]).astype(np.int64)
    rl2, _, _ = _gpu_loss(lp[tok], lpr[tok], A[perm], off2, cuda)
    assert same_bits(rl[torch.from_numpy(perm).to(cuda)], rl2)


def test_response_loss_across_the_tree_boundaries(cuda):
    """Responses just below, at and above the lengths where the sum changes
    tree (one lane / one wavefront / one workgroup) and where it is cut into
    segments (one, two, several), mixed with others: parity with the oracle,
    and each response's loss has the same bits alone, in the batch, and in a
    permuted sub-batch."""
    lane, wave, seg, _ = _loss_constants()
    lens = [1, lane - 1, lane, lane + 1, 63, 64, 65, wave - 1, wave, wave + 1, 1000, seg - 1, seg, seg + 1,
            2 * seg - 1, 2 * seg, 2 * seg + 1, 2 * seg + lane, 2 * seg + wave + 1, 5 * seg + 7, 7]
    rng = np.random.default_rng(21)
    T = np.array(lens * 3)
    N = T.size
    off = np.concatenate([[0], np.cumsum(T)]).astype(np.int64)
    lp = -np.abs(rng.normal(6, 2, off[-1])).astype(np.float32)
    lpr = (lp + rng.normal(0, 0.05, off[-1])).astype(np.float32)
    A = rng.normal(0, 1, N).astype(np.float32)
    rl, _, _ = _check_loss(lp, lpr, A, off, cuda, "tree boundaries")
    _alone_batch_permuted(lp, lpr, A, off, rl, np.arange(len(lens)), cuda, rng)


@pytest.mark.parametrize("pairs", [40, 300])
def test_long_responses_at_every_window_phase(cuda, pairs):
    """Multi-segment responses starting at many offsets relative to the token
    pass's 2048-token windows (short fillers shift them): parity and the same
    bits alone, in the batch and permuted. With 600 responses the batch finds
    each window's responses through the window map, alone through the search
    of the offsets: the two must agree bit for bit."""
    lane, wave, seg, _ = _loss_constants()
    rng = np.random.default_rng(33 + pairs)
    lens = []
    for k in range(pairs):
        lens.append(int(rng.integers(1, seg)))             # a filler that shifts the phase
        lens.append(int(rng.integers(seg + 1, 4 * seg)))    # two to four segments
    T = np.array(lens)
    off = np.concatenate([[0], np.cumsum(T)]).astype(np.int64)
    lp = -np.abs(rng.normal(6, 2, off[-1])).astype(np.float32)
    lpr = (lp + rng.normal(0, 0.05, off[-1])).astype(np.float32)
    A = rng.normal(0, 1, T.size).astype(np.float32)
    rl, _, _ = _check_loss(lp, lpr, A, off, cuda, f"window phases, {T.size} responses")
    _alone_batch_permuted(lp, lpr, A, off, rl, np.arange(1, T.size, 2)[:12], cuda, rng)


def test_loss_millions_of_responses(cuda):
    """About 4.3M responses, mostly of 1-8 tokens, with some of 9-256, of
    257-2048 and of several 2048-token segments, placed across the mean's
    1024-response chunks and the token pass's windows: the per-response
    losses of a sample against the oracle (called on that sample: a
    response's loss depends on it alone), the loss against the mean of the
    float64 per-response losses of the whole batch (the definition, summed
    with numpy), bits alone vs in the batch, and run-to-run bits of the loss."""
    import torch

    lane, wave, seg, chunk = _loss_constants()
    rng = np.random.default_rng(43)
    N = 4_300_000
    T = rng.integers(1, 9, N)
    mid = rng.choice(N, 3000, replace=False)
    T[mid] = rng.integers(9, wave + 1, mid.size)
    big = rng.choice(N, 400, replace=False)
    T[big] = rng.integers(wave + 1, seg + 1, big.size)
    huge = rng.choice(N, 60, replace=False)
    T[huge] = rng.integers(seg + 1, 6 * seg, huge.size)
    # responses straddling the mean's chunk boundaries
    edge = np.concatenate([np.arange(k * chunk - 2, k * chunk + 2) for k in range(1, N // chunk, 997)])
    T[edge] = rng.integers(1, 3 * seg, edge.size)
    off = np.concatenate([[0], np.cumsum(T)]).astype(np.int64)
    n_tok = int(off[-1])
    lp = -np.abs(rng.normal(5, 2, n_tok)).astype(np.float32)
    lpr = (lp + rng.normal(0, 0.1, n_tok)).astype(np.float32)
    A = rng.normal(0, 1, N).astype(np.float32)
    say(f"[loss 4.3M] N={N} n_tok={n_tok}")
    rl, L, c = _gpu_loss(lp, lpr, A, off, cuda)
    _, L2, _ = _gpu_loss(lp, lpr, A, off, cuda)
    assert same_bits(L, L2)
    rl_h = rl.cpu().numpy()
    # a sample: every long response, the chunk-edge ones and random others
    sample = np.unique(np.concatenate([mid[:200], big, huge, edge, rng.choice(N, 2000, replace=False)]))
    tok = np.concatenate([np.arange(off[i], off[i + 1]) for i in sample])
    off_s = np.concatenate([[0], np.cumsum(T[sample])]).astype(np.int64)
    import oracle

    rl_o, _, _ = oracle.reinforce_zero_loss(lp[tok].astype(np.float64), lpr[tok].astype(np.float64),
                                            A[sample].astype(np.float64), off_s)
    e1 = float(rel_err(rl_h[sample], rl_o).max())
    # the loss: the mean of the float64 per-response losses, by definition
    ratio = np.exp(lp.astype(np.float64) - lpr.astype(np.float64))
    l64 = -A.astype(np.float64) * np.add.reduceat(ratio, off[:-1]) / T
    L_o = l64.sum() / N
    e2 = float(rel_err([L.item()], [L_o]).max())
    say(f"[loss 4.3M] rel resp_loss (sample of {sample.size})={e1:.2e} loss={e2:.2e} (|L|={abs(L_o):.3e})")
    assert e1 <= TOL_REL and e2 <= TOL_REL
    _alone_batch_permuted(lp, lpr, A, off, rl, np.concatenate([huge[:8], big[:8], edge[:8], mid[:8]]), cuda, rng)


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
