"""itl_lmhead_logprob_noalloc, called through the C ABI: the same logprob and
lse bits as itl_lmhead_logprob with a caller workspace, on two calls in a
row that share the library's static scratch (the second smaller, so stale
values from the first are still in it), then on the largest call the
scratch holds."""

import ctypes

import pytest

from helpers import same_bits, say

pytestmark = pytest.mark.gpu


def _head(n_tok, d, vocab, seed, device):
    import torch

    g = torch.Generator(device="cpu").manual_seed(seed)
    H = torch.randn(n_tok, d, generator=g).to(torch.bfloat16).to(device)
    W = (torch.randn(vocab, d, generator=g) * 0.02).to(torch.bfloat16).to(device)
    y = torch.randint(0, vocab, (n_tok,), generator=g, dtype=torch.int32).to(device)
    return H, W, y


def _with_workspace(itl, H, W, y):
    import torch

    n_tok, d = H.shape
    vocab = W.shape[0]
    lp = torch.empty(n_tok, dtype=torch.float32, device=H.device)
    lse = torch.empty(n_tok, dtype=torch.float32, device=H.device)
    ws = torch.empty(itl.lmhead_workspace_bytes(n_tok, vocab), dtype=torch.uint8, device=H.device)
    st = itl.lib.itl_lmhead_logprob(ctypes.c_void_p(H.data_ptr()), ctypes.c_void_p(W.data_ptr()), 0, n_tok, d, vocab,
                                    ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(lp.data_ptr()),
                                    ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                    ctypes.c_void_p(torch.cuda.current_stream(H.device).cuda_stream))
    assert st == 0, itl.lib.itl_last_error()
    return lp, lse


def _noalloc(itl, H, W, y):
    import torch

    n_tok, d = H.shape
    vocab = W.shape[0]
    lp = torch.full((n_tok,), float("nan"), dtype=torch.float32, device=H.device)
    lse = torch.full((n_tok,), float("nan"), dtype=torch.float32, device=H.device)
    st = itl.lib.itl_lmhead_logprob_noalloc(ctypes.c_void_p(H.data_ptr()), ctypes.c_void_p(W.data_ptr()), 0, n_tok,
                                            d, vocab, ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(lp.data_ptr()),
                                            ctypes.c_void_p(lse.data_ptr()),
                                            ctypes.c_void_p(torch.cuda.current_stream(H.device).cuda_stream))
    assert st == 0, itl.lib.itl_last_error()
    return lp, lse


@pytest.mark.parametrize("sizes", [(5000, 37), (300, 1)])
def test_noalloc_matches_workspace_call_twice(cuda, sizes):
    import torch
    import invariant_token_logprobs_lm_amd as itl

    vocab, d = 151936, 256
    for k, n_tok in enumerate(sizes):
        H, W, y = _head(n_tok, d, vocab, seed=100 + k + n_tok, device=cuda)
        lp_w, lse_w = _with_workspace(itl, H, W, y)
        lp_n, lse_n = _noalloc(itl, H, W, y)
        torch.cuda.synchronize()
        say(f"[noalloc] call {k}: n_tok={n_tok} vocab={vocab} d={d}")
        assert same_bits(lp_n, lp_w) and same_bits(lse_n, lse_w), (k, n_tok)


def test_noalloc_largest_call_then_a_small_one(cuda):
    import torch
    import invariant_token_logprobs_lm_amd as itl

    vocab, d = 151936, 128
    for k, n_tok in enumerate((16368, 65)):
        H, W, y = _head(n_tok, d, vocab, seed=7 + k, device=cuda)
        lp_w, lse_w = _with_workspace(itl, H, W, y)
        lp_n, lse_n = _noalloc(itl, H, W, y)
        torch.cuda.synchronize()
        say(f"[noalloc] n_tok={n_tok}")
        assert same_bits(lp_n, lp_w) and same_bits(lse_n, lse_w), n_tok
    # one token more than the scratch holds: refused before any launch
    H, W, y = _head(16369, d, vocab, seed=9, device=cuda)
    st = itl.lib.itl_lmhead_logprob_noalloc(ctypes.c_void_p(H.data_ptr()), ctypes.c_void_p(W.data_ptr()), 0, 16369,
                                            d, vocab, ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(1), None, None)
    assert st == 2 and b"scratch" in itl.lib.itl_last_error()
