"""The forward logprob and the loss under HIP graph capture: a serving loop
can capture a decode step (and a prefill) once and replay it. Every replay,
with eager work and synchronisations in between, must give the eager
result's bits (the path records no memset node: the library clears nothing
in device memory)."""

import numpy as np
import pytest

from helpers import same_bits

pytestmark = pytest.mark.gpu


def _head(n_tok, d, vocab, seed, device):
    import torch

    g = torch.Generator(device="cpu").manual_seed(seed)
    H = torch.randn(n_tok, d, generator=g).to(torch.bfloat16).to(device)
    W = (torch.randn(vocab, d, generator=g) * 0.02).to(torch.bfloat16).to(device)
    y = torch.randint(0, vocab, (n_tok,), generator=g, dtype=torch.int32).to(device)
    return H, W, y


@pytest.mark.parametrize("n_tok", [8, 1000])   # the narrow (decode) and the wide kernel
def test_logprob_and_loss_replay(cuda, n_tok):
    import torch
    import invariant_token_logprobs_lm_amd as itl

    H, W, y = _head(n_tok, 512, 20000, seed=n_tok, device=cuda)
    ws = torch.empty(itl.lmhead_workspace_bytes(n_tok, 20000), dtype=torch.uint8, device=cuda)
    lp = torch.empty(n_tok, dtype=torch.float32, device=cuda)
    lse = torch.empty(n_tok, dtype=torch.float32, device=cuda)
    lpr = torch.zeros(n_tok, dtype=torch.float32, device=cuda)
    roff = torch.tensor([0, n_tok // 2, n_tok], dtype=torch.int64, device=cuda)
    A = torch.tensor([0.5, -0.5], dtype=torch.float32, device=cuda)
    # eager reference
    lp_e, lse_e = itl.lmhead_logprob(H, W, y)
    rl_e, L_e, c_e = itl.reinforce_zero_loss(lp_e, lpr, A, roff)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=cuda)
    side.wait_stream(torch.cuda.current_stream(cuda))
    with torch.cuda.stream(side):  # warm up on the capture stream
        itl.lmhead_logprob(H, W, y, logprob=lp, lse=lse, workspace=ws)
    torch.cuda.current_stream(cuda).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        itl.lmhead_logprob(H, W, y, logprob=lp, lse=lse, workspace=ws)
        rl, L, c = itl.reinforce_zero_loss(lp, lpr, A, roff)
    for rep in range(4):
        lp.fill_(float("nan"))
        lse.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert same_bits(lp, lp_e) and same_bits(lse, lse_e), rep
        assert same_bits(rl, rl_e) and same_bits(L, L_e) and same_bits(c, c_e), rep
        # eager work between replays on the same memory
        itl.lmhead_logprob(H[: max(1, n_tok // 3)], W, y[: max(1, n_tok // 3)])
        torch.cuda.synchronize()
