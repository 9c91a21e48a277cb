"""The forward logprob, the loss and the mismatch diagnostics under HIP graph
capture: a serving loop can capture a decode step (and a prefill) once and
replay it. Every replay, with eager work and synchronisations in between,
must give the eager result's bits (the path records no memset node: what
the library clears in device memory, it clears with a kernel)."""

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


def test_mismatch_stats_replay(cuda):
    """The diagnostics clear their own histogram with a kernel: every replay,
    with an eager call on other data dirtying the same workspace in between,
    gives the eager result's bits."""
    import torch
    import invariant_token_logprobs_lm_amd as itl

    n = 50_000
    rng = np.random.default_rng(5)
    lp = torch.from_numpy(-np.abs(rng.standard_normal(n)).astype(np.float32)).to(cuda)
    lr = lp + torch.from_numpy(rng.normal(0, 0.05, n).astype(np.float32)).to(cuda)
    other = lp + torch.from_numpy(rng.normal(0, 1.0, n).astype(np.float32)).to(cuda)
    ws = torch.empty(itl.mismatch_stats_workspace_bytes(n), dtype=torch.uint8, device=cuda)
    st = torch.empty(len(itl.STAT_FIELDS), dtype=torch.float64, device=cuda)
    ref = itl.mismatch_stats(lp, lr).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=cuda)
    side.wait_stream(torch.cuda.current_stream(cuda))
    with torch.cuda.stream(side):
        itl.mismatch_stats(lp, lr, stats=st, workspace=ws)
    torch.cuda.current_stream(cuda).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        itl.mismatch_stats(lp, lr, stats=st, workspace=ws)
    for rep in range(4):
        st.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.view(torch.int64), ref.view(torch.int64)), rep
        itl.mismatch_stats(lp, other, workspace=ws)  # eager call on other data, same workspace
        torch.cuda.synchronize()
