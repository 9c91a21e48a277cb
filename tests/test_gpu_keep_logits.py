"""GPU tests of the kept-logits forward and the backward that reads them.

itl_lmhead_logprob_keep_logits must give the same logprob and lse bits as
itl_lmhead_logprob and write every logit z[t, v] within the logprob bar of
the float64 oracle's (|dz| <= 1e-3; the fp32 accumulators are far closer);
entries past the vocabulary in a padded row stay untouched.
itl_reinforce_zero_backward_from_logits must give dH and dW with the same
bits as itl_reinforce_zero_backward (which the backward parity tests pin to
the oracle), and on its own be within 1e-3 (Frobenius-relative) of the
oracle. Cases: the narrow (<= 64 tokens) and wide kernels, ragged vocabulary
tails (vocab not a multiple of 4 or of the 256-row tile), a padded row
stride, the fp32 head, two token chunks of the backward, and the large-MoE
head at full size (the benchmark's launches).
"""

import numpy as np
import pytest

from helpers import host_array, same_bits, say

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _itl():
    import invariant_token_logprobs_lm_amd as itl

    return itl


def _random_head(n_tok, d, vocab, dtype, seed, device, w_std=0.05):
    import torch

    g = torch.Generator(device="cpu").manual_seed(seed)
    H = torch.randn(n_tok, d, generator=g).to(dtype)
    W = (torch.randn(vocab, d, generator=g) * w_std).to(dtype)
    y = torch.randint(0, vocab, (n_tok,), generator=g, dtype=torch.int32)
    return H.to(device), W.to(device), y.to(device)


@pytest.mark.parametrize(
    "n_tok,d,vocab,pad,dtype_name",
    [
        (40, 128, 1000, 0, "bf16"),          # narrow kernel, vocab a multiple of 4 but not of 256
        (64, 256, 4096 + 37, 12, "bf16"),    # narrow, last tile of 37 rows, vocab not a multiple of 4, padded rows
        (65, 192, 3001, 3, "bf16"),          # the 128-token narrow block from 65 tokens on, 1 row past 64
        (128, 64, 1030, 2, "f32"),           # a full 128-token narrow block, fp32 head
        (129, 192, 3001, 0, "bf16"),         # the wide kernel from 129 tokens on
        (700, 256, 5000, 0, "bf16"),         # 3 token blocks (ragged), 20 vocabulary tiles
        (300, 64, 1030, 2, "f32"),           # fp32 head
    ],
)
def test_keep_logits_forward(cuda, n_tok, d, vocab, pad, dtype_name):
    import torch
    import oracle

    itl = _itl()
    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    H, W, y = _random_head(n_tok, d, vocab, dt, seed=n_tok * 13 + vocab, device=cuda)
    ld = (vocab + 3) // 4 * 4 + 4 * pad
    sentinel = -12345.0
    Z = torch.full((n_tok, ld), sentinel, dtype=torch.float32, device=cuda)
    lp_k, lse_k, _ = itl.lmhead_logprob_keep_logits(H, W, y, logits=Z)
    lp, lse = itl.lmhead_logprob(H, W, y)
    torch.cuda.synchronize()
    say(f"[keep {n_tok}x{d}x{vocab} ld={ld} {dtype_name}]")
    assert same_bits(lp_k, lp) and same_bits(lse_k, lse)
    z_o = oracle.logits(host_array(H), host_array(W))
    Zh = Z.cpu().numpy()
    err = float(np.max(np.abs(Zh[:, :vocab].astype(np.float64) - z_o)))
    say(f"  max |z - z_oracle| = {err:.2e}")
    assert err <= TOL
    assert bool((Z[:, vocab:] == sentinel).all())


def test_keep_logits_rejects_bad_stride(cuda):
    import torch

    itl = _itl()
    H, W, y = _random_head(8, 64, 100, torch.bfloat16, seed=1, device=cuda)
    for ld in (96, 102):  # below vocab; not a multiple of 4
        with pytest.raises(itl.ItlError):
            itl.lmhead_logprob_keep_logits(H, W, y, logits=torch.empty((8, ld), dtype=torch.float32, device=cuda))


def _loss_coef(lp, rng, n):
    """Per-token coefficients of the loss for a random response layout."""
    import torch

    itl = _itl()
    dev = lp.device
    n_resp = max(1, n // 37)
    cuts = np.sort(rng.choice(np.arange(1, n), size=n_resp - 1, replace=False)) if n_resp > 1 else np.array([], int)
    roff = torch.as_tensor(np.concatenate([[0], cuts, [n]]).astype(np.int64), device=dev)
    goff = np.arange(0, n_resp + 1, 4, dtype=np.int32)
    if goff[-1] != n_resp:
        goff = np.append(goff, n_resp).astype(np.int32)
    goff = torch.as_tensor(goff, device=dev)
    rewards = torch.as_tensor(rng.random(n_resp).astype(np.float32), device=dev)
    lpr = lp + torch.as_tensor(rng.normal(0, 0.02, n).astype(np.float32), device=dev)
    A = itl.group_advantage(rewards, goff)
    return itl.reinforce_zero_loss(lp, lpr, A, roff)[2]


@pytest.mark.parametrize(
    "n_tok,d,vocab,dtype_name",
    [
        (700, 256, 5000, "bf16"),
        (300, 128, 4096 + 37, "bf16"),
        (257, 64, 1000, "f32"),
        (1, 192, 300, "bf16"),
        (16384 + 300, 128, 2000, "bf16"),  # two chunks of the backward
    ],
)
def test_backward_from_logits_matches_recompute(cuda, n_tok, d, vocab, dtype_name):
    import torch
    import oracle

    itl = _itl()
    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    H, W, y = _random_head(n_tok, d, vocab, dt, seed=n_tok * 3 + d, device=cuda)
    if n_tok > 16384:
        y[::3] = 7
    lp, lse, Z = itl.lmhead_logprob_keep_logits(H, W, y)
    coef = _loss_coef(lp, np.random.default_rng(n_tok), n_tok)
    dH_k, dW_k = itl.reinforce_zero_backward_from_logits(H, W, y, lse, coef, Z)
    dH_r, dW_r = itl.reinforce_zero_backward(H, W, y, lse, coef)
    torch.cuda.synchronize()
    say(f"[backward from logits {n_tok}x{d}x{vocab} {dtype_name}]")
    assert same_bits(dH_k, dH_r) and same_bits(dW_k, dW_r)
    if n_tok <= 1000:
        Hh, Wh, yh = host_array(H), host_array(W), y.cpu().numpy()
        dH_o, dW_o = oracle.reinforce_zero_backward(Hh, Wh, yh, coef.cpu().numpy().astype(np.float64))
        for got, want, name in ((dH_k, dH_o, "dH"), (dW_k, dW_o, "dW")):
            g = got.cpu().numpy().astype(np.float64)
            e = float(np.linalg.norm(g - want) / max(np.linalg.norm(want), 1e-300))
            say(f"  fro rel {name} = {e:.2e}")
            assert e <= TOL


def test_keep_logits_large_moe_head_full_size(cuda):
    """The benchmark's forward + backward on the large-MoE head at full size
    (308,010 tokens, 159 GB of kept logits): logprobs bit-identical to the
    plain forward, dH and dW bit-identical to the recomputing backward."""
    import torch
    from synth import WORKLOADS, draw_head, draw_layout, sample_tokens

    itl = _itl()
    wl = WORKLOADS["large-moe-head"]
    lay = draw_layout(wl)
    n = lay.n_tok
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info(cuda)
    need = n * wl.vocab * 4 + 2 * n * wl.d * 4 + (40 << 30)
    if free < need:
        pytest.skip(f"needs about {need / 2**30:.0f} GiB free, {free / 2**30:.0f} GiB available")
    say(f"[keep full] n_tok={n} d={wl.d} V={wl.vocab}")
    H, W = draw_head(wl, n, device=cuda)
    y = sample_tokens(H, W, wl)
    lp, lse, Z = itl.lmhead_logprob_keep_logits(H, W, y)
    lp2, lse2 = itl.lmhead_logprob(H, W, y)
    torch.cuda.synchronize()
    assert same_bits(lp, lp2) and same_bits(lse, lse2)
    coef = _loss_coef(lp, np.random.default_rng(11), n)
    dH_k, dW_k = itl.reinforce_zero_backward_from_logits(H, W, y, lse, coef, Z)
    del Z
    dH_r, dW_r = itl.reinforce_zero_backward(H, W, y, lse, coef)
    torch.cuda.synchronize()
    assert same_bits(dH_k, dH_r) and same_bits(dW_k, dW_r)


def test_kept_logits_are_batch_invariant(cuda):
    """A token's kept logits have the same bits alone (narrow kernel), in a
    small batch, and in a large batch at another row position (wide kernel),
    so the dlogits formed from them are batch-invariant per token too."""
    import torch

    itl = _itl()
    H, W, y = _random_head(900, 256, 3000, torch.bfloat16, seed=77, device=cuda)
    _, _, Z_all = itl.lmhead_logprob_keep_logits(H, W, y)
    pick = [0, 5, 257, 600, 899]
    idx = torch.tensor(pick, device=cuda)
    _, _, Z_few = itl.lmhead_logprob_keep_logits(H[idx].contiguous(), W, y[idx].contiguous())
    perm = torch.randperm(900, generator=torch.Generator(device="cpu").manual_seed(3)).to(cuda)
    _, _, Z_perm = itl.lmhead_logprob_keep_logits(H[perm].contiguous(), W, y[perm].contiguous())
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(900, device=cuda)
    torch.cuda.synchronize()
    for k, t in enumerate(pick):
        _, _, Z_one = itl.lmhead_logprob_keep_logits(H[t:t + 1].contiguous(), W, y[t:t + 1].contiguous())
        torch.cuda.synchronize()
        assert same_bits(Z_one[0, :3000], Z_all[t, :3000])
        assert same_bits(Z_few[k, :3000], Z_all[t, :3000])
        assert same_bits(Z_perm[inv[t], :3000], Z_all[t, :3000])
