"""GPU parity of itl_reinforce_zero_backward against the float64 oracle.

Bar: dH and dW within 1e-3 relative to the oracle in Frobenius norm, per
tensor (the largest row-wise relative error is printed, not gated). The GPU
runs the whole path (forward logprob, advantage, loss with its per-token
coefficients, backward) on the same input bits the oracle reads; the oracle
computes its own logprobs and coefficients in float64. Cases span several
tiles, ragged tails in every dimension, tokens sharing an id, several token
chunks, the tiny fp32 head, and the large-MoE head shape (reduced token
count, sampled rows). Run-to-run bit equality of dH and dW is checked too.
"""

import re

import numpy as np
import pytest

from helpers import host_array, same_bits, say

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _itl():
    import invariant_token_logprobs_lm_amd as itl

    return itl


def _fro_rel(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))


def _row_rel_max(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    num = np.linalg.norm(got - want, axis=1)
    den = np.maximum(np.linalg.norm(want, axis=1), 1e-300)
    return float(np.max(num / den))


def _gpu_path(H, W, y, lpr_noise, rewards, goff, roff):
    """Forward + advantage + loss + backward on the GPU; returns tensors."""
    import torch

    itl = _itl()
    dev = H.device
    lp, lse = itl.lmhead_logprob(H, W, y)
    lpr = lp + torch.as_tensor(lpr_noise, device=dev)
    A = itl.group_advantage(torch.as_tensor(rewards, device=dev), torch.as_tensor(goff, device=dev))
    rl, L, coef = itl.reinforce_zero_loss(lp, lpr, A, torch.as_tensor(roff, device=dev))
    dH, dW = itl.reinforce_zero_backward(H, W, y, lse, coef)
    torch.cuda.synchronize()
    return lp, lpr, coef, dH, dW


def _oracle_coef(Hh, Wh, yh, lpr, rewards, goff, roff):
    import oracle

    lp_o, _ = oracle.lmhead_logprob(Hh, Wh, yh)
    A_o = oracle.group_advantage(rewards, goff)
    _, _, c_o = oracle.reinforce_zero_loss(lp_o, lpr, A_o, roff)
    return c_o


def _check_full(H, W, y, rng, lag=0.02, label=""):
    """Compare every element of dH and dW with the oracle."""
    import oracle

    n = H.shape[0]
    n_resp = max(1, n // 37)
    rewards = rng.random(n_resp).astype(np.float32)
    # spread n tokens over n_resp responses (groups of 4)
    cuts = np.sort(rng.choice(np.arange(1, n), size=n_resp - 1, replace=False)) if n_resp > 1 else np.array([], int)
    roff = np.concatenate([[0], cuts, [n]]).astype(np.int64)
    goff = np.arange(0, n_resp + 1, 4, dtype=np.int32)
    if goff[-1] != n_resp:
        goff = np.append(goff, n_resp).astype(np.int32)
    noise = rng.normal(0, lag, n).astype(np.float32)
    lp, lpr, coef, dH, dW = _gpu_path(H, W, y, noise, rewards, goff, roff)
    Hh, Wh, yh = host_array(H), host_array(W), y.cpu().numpy()
    # the oracle's rollout record: the GPU's record bits (same input for both sides)
    lpr_h = lpr.cpu().numpy().astype(np.float64)
    c_o = _oracle_coef(Hh, Wh, yh, lpr_h, rewards.astype(np.float64), goff, roff)
    dH_o, dW_o = oracle.reinforce_zero_backward(Hh, Wh, yh, c_o)
    eH = _fro_rel(dH.cpu().numpy(), dH_o)
    eW = _fro_rel(dW.cpu().numpy(), dW_o)
    say(f"[backward {label}] n={n} d={H.shape[1]} V={W.shape[0]} {H.dtype}: fro rel dH={eH:.2e} dW={eW:.2e} "
        f"(max row rel dH={_row_rel_max(dH.cpu().numpy(), dH_o):.2e})")
    assert eH <= TOL and eW <= TOL
    # run-to-run determinism
    itl = _itl()
    import torch

    lse = itl.lmhead_logprob(H, W, y)[1]
    dH2, dW2 = itl.reinforce_zero_backward(H, W, y, lse, coef)
    dH3, dW3 = itl.reinforce_zero_backward(H, W, y, lse, coef)
    lp2, lse2 = itl.lmhead_logprob(H, W, y)
    torch.cuda.synchronize()
    assert same_bits(dH2, dH3) and same_bits(dW2, dW3)
    assert same_bits(dH, dH2) and same_bits(dW, dW2)


def _random_head(n_tok, d, vocab, dtype, seed, device, w_std=0.05):
    import torch

    g = torch.Generator(device="cpu").manual_seed(seed)
    H = torch.randn(n_tok, d, generator=g).to(dtype)
    W = (torch.randn(vocab, d, generator=g) * w_std).to(dtype)
    y = torch.randint(0, vocab, (n_tok,), generator=g, dtype=torch.int32)
    return H.to(device), W.to(device), y.to(device)


def test_tiny_workload_backward(cuda):
    import torch
    import oracle
    from synth import WORKLOADS, draw_head, draw_layout, sample_tokens

    wl = WORKLOADS["tiny"]
    lay = draw_layout(wl)
    H, W = draw_head(wl, lay.n_tok, device="cpu")
    y = sample_tokens(H, W, wl)
    Hd, Wd, yd = H.to(cuda), W.to(cuda), y.to(cuda)
    lp, lpr, coef, dH, dW = _gpu_path(Hd, Wd, yd, lay.lag_noise, lay.rewards, lay.group_offsets, lay.resp_offsets)
    c_o = _oracle_coef(H.numpy(), W.numpy(), y.numpy(), lpr.cpu().numpy().astype(np.float64),
                       lay.rewards.astype(np.float64), lay.group_offsets, lay.resp_offsets)
    dH_o, dW_o = oracle.reinforce_zero_backward(H.numpy(), W.numpy(), y.numpy(), c_o)
    eH, eW = _fro_rel(dH.cpu().numpy(), dH_o), _fro_rel(dW.cpu().numpy(), dW_o)
    say(f"[backward tiny] n={lay.n_tok}: fro rel dH={eH:.2e} dW={eW:.2e}")
    assert eH <= TOL and eW <= TOL


@pytest.mark.parametrize(
    "n_tok,d,vocab,dtype_name",
    [
        (700, 256, 5000, "bf16"),         # 3 token blocks (ragged), 20 vocabulary tiles, ragged tail
        (300, 128, 4096 + 37, "bf16"),    # last vocabulary tile of 37 rows
        (257, 64, 1000, "f32"),           # fp32 path, one K step per row
        (1, 192, 300, "bf16"),            # a single token
        (513, 320, 8192 + 256, "bf16"),   # d not a multiple of the 256-row tile
        (300, 3136, 2000, "bf16"),        # 49 K steps: the recomputed logits' token block two steps ahead
    ],
)
def test_backward_shapes(cuda, n_tok, d, vocab, dtype_name):
    import torch

    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    H, W, y = _random_head(n_tok, d, vocab, dt, seed=n_tok * 7 + vocab, device=cuda)
    _check_full(H, W, y, np.random.default_rng(n_tok), label=f"{n_tok}x{d}x{vocab}")


def test_backward_repeated_ids_and_several_chunks(cuda):
    """More tokens than one chunk (16384), many sharing a few ids."""
    import torch

    H, W, y = _random_head(16384 + 300, 128, 2000, torch.bfloat16, seed=99, device=cuda)
    y[::3] = 7           # a long run of one id, spread over both chunks
    y[1::50] = 1999      # the last vocabulary row
    _check_full(H, W, y, np.random.default_rng(5), label="two chunks, repeated ids")


def test_backward_large_moe_head_rows(cuda):
    """The large-MoE head (d=7168, V=129280) on a reduced-token instance: one
    group of 16 responses of 8..32 tokens; the oracle recomputes sampled rows
    of dH and dW (every token's softmax over the full vocabulary)."""
    import torch
    import oracle
    from synth import WORKLOADS, draw_head, draw_layout, sample_tokens, token_subset

    wl = WORKLOADS["large-moe-head"]
    lay = draw_layout(wl, n_groups=1, group_size=16, len_lo=8, len_hi=32, salt=1)
    H, W = draw_head(wl, lay.n_tok, device=cuda, salt=1)
    y = sample_tokens(H, W, wl, salt=1)
    say(f"[backward large-moe] n_tok={lay.n_tok}")
    lp, lpr, coef, dH, dW = _gpu_path(H, W, y, lay.lag_noise, lay.rewards, lay.group_offsets, lay.resp_offsets)
    Hh, Wh, yh = host_array(H), host_array(W), y.cpu().numpy()
    c_o = _oracle_coef(Hh, Wh, yh, lpr.cpu().numpy().astype(np.float64), lay.rewards.astype(np.float64),
                       lay.group_offsets, lay.resp_offsets)
    tok = token_subset(lay.n_tok, 24, seed=7)
    voc = np.unique(np.concatenate([yh[tok[:8]], token_subset(wl.vocab, 24, seed=8)]))
    dH_o, dW_o = oracle.reinforce_zero_backward_rows(Hh, Wh, yh, c_o, tok, voc)
    eH = _fro_rel(dH.cpu().numpy()[tok], dH_o)
    eW = _fro_rel(dW.cpu().numpy()[voc], dW_o)
    say(f"[backward large-moe] sampled rows: fro rel dH={eH:.2e} dW={eW:.2e}")
    assert eH <= TOL and eW <= TOL


def test_backward_full_size_determinism(cuda):
    """The large-MoE head at full size (the benchmark's backward launch):
    finite, run-to-run bit-identical, every column of dW sums to about zero
    over the vocabulary (each token's dlogits sum to zero), and dH rows of
    tokens in every one of the backward's token chunks match the oracle
    (given the GPU's coefficients: a dH row needs only its own token's
    log-normaliser over the full vocabulary)."""
    import torch
    from synth import WORKLOADS, draw_head, draw_layout, sample_tokens

    wl = WORKLOADS["large-moe-head"]
    lay = draw_layout(wl)
    say(f"[backward full] n_tok={lay.n_tok} d={wl.d} V={wl.vocab}")
    H, W = draw_head(wl, lay.n_tok, device=cuda)
    y = sample_tokens(H, W, wl)
    lp, lpr, coef, dH, dW = _gpu_path(H, W, y, lay.lag_noise, lay.rewards, lay.group_offsets, lay.resp_offsets)
    assert bool(torch.isfinite(dH).all()) and bool(torch.isfinite(dW).all())
    itl = _itl()
    lse = itl.lmhead_logprob(H, W, y)[1]
    dH2, dW2 = itl.reinforce_zero_backward(H, W, y, lse, coef)
    torch.cuda.synchronize()
    assert same_bits(dH, dH2) and same_bits(dW, dW2)
    colsum = dW.double().sum(dim=0).abs().max().item()
    scale = dW.double().abs().sum(dim=0).max().item()
    say(f"[backward full] max |column sum of dW| = {colsum:.3e} (column abs-sum up to {scale:.3e})")
    assert colsum <= 1e-2 * scale
    import oracle

    chunk = int(re.search(r"bwd_chunk_tokens=(\d+)", itl.build_info()).group(1))
    rng = np.random.default_rng(21)
    n = lay.n_tok
    tok = [int(rng.integers(c0, min(n, c0 + chunk))) for c0 in range(0, n, chunk)]
    tok = np.unique(np.concatenate([tok, rng.choice(n, size=24 - len(tok) if len(tok) < 24 else 0, replace=False)]))
    tt = torch.as_tensor(tok, device=cuda)
    dH_o, _ = oracle.reinforce_zero_backward_rows(host_array(H.index_select(0, tt)), host_array(W),
                                                   y.index_select(0, tt).cpu().numpy(),
                                                   coef.index_select(0, tt).cpu().numpy().astype(np.float64),
                                                   np.arange(len(tok)), np.zeros(0, np.int64))
    eH = _fro_rel(dH.index_select(0, tt).cpu().numpy(), dH_o)
    say(f"[backward full] {len(tok)} dH rows over {(n + chunk - 1) // chunk} chunks: fro rel {eH:.2e} "
        f"(max row rel {_row_rel_max(dH.index_select(0, tt).cpu().numpy(), dH_o):.2e})")
    assert eH <= TOL


def _zipf_ids(n, vocab, rng, hot, share):
    """Token ids with one id taking `share` of the tokens and the rest
    Zipf-like (id k drawn with weight 1 / (k + 1)), as sampled text gives."""
    w = 1.0 / np.arange(1, vocab + 1)
    y = rng.choice(vocab, size=n, p=w / w.sum()).astype(np.int32)
    y[rng.random(n) < share] = hot
    return y


def test_backward_zipf_tokens(cuda):
    """Zipf-like ids with one id at about 35 % of the tokens (a run of
    several thousand tokens: several segment groups in the sampled term),
    over two token chunks: oracle parity and run-to-run bits."""
    import torch

    rng = np.random.default_rng(11)
    H, W, _ = _random_head(20000, 128, 3000, torch.bfloat16, seed=123, device=cuda)
    y = _zipf_ids(20000, 3000, rng, hot=1234, share=0.35)
    say(f"[backward zipf] hot id share {(y == 1234).mean():.3f}, distinct ids {len(np.unique(y))}")
    _check_full(H, W, torch.as_tensor(y, device=cuda), np.random.default_rng(6), label="zipf")


def _emulate_sampled_rows(Hf, y, c, vocab, seg=64, group=64):
    """dW's sampled term in the library's documented order, in float32 with
    every product and sum rounded on its own: each id's tokens in ascending
    order, summed in segments of `seg`, groups of `group` segments, then the
    groups (a run of at most one segment is its own sum)."""
    d = Hf.shape[1]
    out = np.zeros((vocab, d), np.float32)
    c = c.astype(np.float32)
    for v in np.unique(y):
        toks = np.nonzero(y == v)[0]
        sums = []
        for j in range(0, len(toks), seg):
            acc = np.zeros(d, np.float32)
            for t in toks[j:j + seg]:
                acc = acc + c[t] * Hf[t]
            sums.append(acc)
        if len(sums) == 1:
            out[v] = sums[0]
            continue
        groups = []
        for g in range(0, len(sums), group):
            acc = np.zeros(d, np.float32)
            for s in sums[g:g + group]:
                acc = acc + s
            groups.append(acc)
        if len(groups) == 1:
            out[v] = groups[0]
            continue
        acc = np.zeros(d, np.float32)
        for s in groups:
            acc = acc + s
        out[v] = acc
    return out


def test_sampled_term_follows_its_order(cuda):
    """With lse far above every logit the dense part of the dlogits is
    exactly zero, so dW is the sampled term alone and dH the sampled rows
    coef[t] W[y_t]: both must equal, value for value, a float32 emulation of
    the documented order (runs of 6,000 tokens: two groups; 500: one group of
    8 segments; 65 and 64 tokens; single tokens; rows no token samples are
    zero). Not an oracle comparison: this pins the summation order itself."""
    import torch

    itl = _itl()
    rng = np.random.default_rng(3)
    n, d, vocab = 12000, 128, 1000
    y = rng.integers(100, vocab, size=n).astype(np.int32)
    pos = rng.permutation(n)
    y[pos[:6000]] = 5
    y[pos[6000:6500]] = 17
    y[pos[6500:6565]] = 31
    y[pos[6565:6629]] = 40
    y[(y >= 500) & (y < 520)] = 499  # ids 500..519 sampled by no token
    H = torch.randn(n, d, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    W = (torch.randn(vocab, d, generator=torch.Generator().manual_seed(5)) * 0.05).to(torch.bfloat16)
    coef = rng.normal(0, 1e-3, n).astype(np.float32)
    lse = np.full(n, 1e4, np.float32)
    dH, dW = itl.reinforce_zero_backward(H.to(cuda), W.to(cuda), torch.as_tensor(y, device=cuda),
                                         torch.as_tensor(lse, device=cuda), torch.as_tensor(coef, device=cuda))
    torch.cuda.synchronize()
    Hf, Wf = H.float().numpy(), W.float().numpy()
    want_W = _emulate_sampled_rows(Hf, y, coef, vocab)
    want_H = np.float32(0) + coef[:, None] * Wf[y]
    got_W, got_H = dW.cpu().numpy(), dH.cpu().numpy()
    bad_rows = np.nonzero(~np.all(got_W == want_W, axis=1))[0]
    say(f"[sampled order] rows differing from the emulation: {len(bad_rows)} {bad_rows[:8]}")
    assert len(bad_rows) == 0
    assert np.array_equal(got_H, want_H)
    assert not got_W[500:520].any()


def test_dh_rows_are_batch_invariant(cuda):
    """dH[t] = sum_v G[t, v] W[v] + coef[t] W[y_t] involves token t alone, and
    each token's column of the contraction is computed by the same
    instruction sequence at any position: given the same lse and coef, a
    token's dH row has the same bits in the full batch, alone, and in a
    permuted sub-batch that straddles the backward's token chunks."""
    import torch

    itl = _itl()
    H, W, y = _random_head(16384 + 700, 256, 3000, torch.bfloat16, seed=77, device=cuda)
    lse = itl.lmhead_logprob(H, W, y)[1]
    coef = torch.as_tensor(np.random.default_rng(8).normal(0, 1e-3, H.shape[0]).astype(np.float32), device=cuda)
    dH, _ = itl.reinforce_zero_backward(H, W, y, lse, coef)
    rng = np.random.default_rng(9)
    pick = np.sort(rng.choice(H.shape[0], 40, replace=False))
    for t in pick[:6]:
        s = slice(int(t), int(t) + 1)
        dH1, _ = itl.reinforce_zero_backward(H[s], W, y[s], lse[s], coef[s])
        assert same_bits(dH1, dH[s]), int(t)
    perm = torch.as_tensor(rng.permutation(np.concatenate([pick, np.arange(16000, 16900)])), device=cuda)
    dH2, _ = itl.reinforce_zero_backward(H[perm].contiguous(), W, y[perm].contiguous(), lse[perm].contiguous(),
                                         coef[perm].contiguous())
    torch.cuda.synchronize()
    assert same_bits(dH2, dH[perm])
