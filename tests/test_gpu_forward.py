"""GPU parity of itl_lmhead_logprob against the float64 oracle.

Bar: |logprob_gpu - logprob_oracle| <= 1e-3 absolute (and the same for lse),
on the same input bits. Small cases compare every token; full-size heads
compare a seeded sample of tokens in the launch configuration the benchmark
uses, plus properties that hold at any size (logprob <= 0 in fp32, run-to-run
bit equality).
"""

import numpy as np
import pytest

from helpers import host_array, same_bits, say

pytestmark = pytest.mark.gpu

TOL_LP = 1e-3


def _itl():
    import invariant_token_logprobs_lm_amd as itl

    return itl


def _random_head(n_tok, d, vocab, dtype, seed, device, w_std=0.02):
    import torch

    g = torch.Generator(device="cpu").manual_seed(seed)
    H = torch.randn(n_tok, d, generator=g).to(dtype)
    W = (torch.randn(vocab, d, generator=g) * w_std).to(dtype)
    y = torch.randint(0, vocab, (n_tok,), generator=g, dtype=torch.int32)
    return H.to(device), W.to(device), y.to(device)


def _parity(H, W, y, tol=TOL_LP, label=""):
    import oracle

    itl = _itl()
    lp, lse = itl.lmhead_logprob(H, W, y)
    lp_o, lse_o = oracle.lmhead_logprob(host_array(H), host_array(W), y.cpu().numpy())
    lp_g = lp.cpu().numpy().astype(np.float64)
    lse_g = lse.cpu().numpy().astype(np.float64)
    e_lp = float(np.max(np.abs(lp_g - lp_o))) if lp_o.size else 0.0
    e_lse = float(np.max(np.abs(lse_g - lse_o))) if lp_o.size else 0.0
    say(f"[parity {label}] n={H.shape[0]} d={H.shape[1]} V={W.shape[0]} {H.dtype}: max|dlp|={e_lp:.3e} max|dlse|={e_lse:.3e}")
    assert e_lp <= tol and e_lse <= tol
    assert np.all(lp_g <= 0.0)
    return lp, lse


def test_tiny_workload_all_tokens(cuda):
    import torch
    from synth import WORKLOADS, draw_head, draw_layout, sample_tokens

    wl = WORKLOADS["tiny"]
    lay = draw_layout(wl)
    H, W = draw_head(wl, lay.n_tok, device="cpu")
    y = sample_tokens(H, W, wl)
    _parity(H.to(cuda), W.to(cuda), y.to(cuda), label="tiny fp32")


@pytest.mark.parametrize(
    "n_tok,d,vocab,dtype_name",
    [
        (700, 256, 5000, "bf16"),    # 3 token blocks (ragged), 20 vocab tiles = 20 slices, ragged tail
        (300, 128, 4096 + 37, "bf16"),  # last tile (and slice) holds 37 rows
        (257, 64, 1000, "f32"),      # one K step per tile, fp32 MFMA
        (1, 192, 300, "bf16"),       # one token
        (5, 64, 1, "bf16"),          # vocabulary of one: logprob = 0 exactly
        (64, 64, 3, "f32"),          # tiny vocabulary, mostly masked tile
        (513, 320, 8192 + 256, "bf16"),  # 33 slices of one tile, d not a multiple of 256
        (5200, 64, 150 * 256 - 17, "bf16"),  # 21 x 150 > 2048: 8 slices per workgroup, last group of 6
        (300, 4160, 3005, "bf16"),   # 65 K steps: the token block staged two K steps ahead
        (300, 3072, 2000, "bf16"),   # 48 K steps: the last length with the token block one step ahead
        (300, 3136, 2000, "bf16"),   # 49 K steps: the first with it two steps ahead
        (260, 32768, 700, "bf16"),   # 256 K steps of 64 KiB rows: the largest d tested
        (300, 2112, 1000, "f32"),    # 66 K steps of fp32: the same ring order, fp32 MFMA
    ],
)
def test_shapes_ragged_and_degenerate(cuda, n_tok, d, vocab, dtype_name):
    import torch

    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    H, W, y = _random_head(n_tok, d, vocab, dt, seed=n_tok * 31 + vocab, device=cuda, w_std=0.2)
    lp, _ = _parity(H, W, y, label=f"{n_tok}x{d}x{vocab}")
    if vocab == 1:
        assert torch.all(lp == 0.0)


def test_sampled_token_at_every_tile_position(cuda):
    """y covers every row of a tile and the first/last vocabulary ids."""
    import torch

    vocab, d = 1024 + 100, 128
    n_tok = 512
    H, W, _ = _random_head(n_tok, d, vocab, torch.bfloat16, seed=7, device=cuda, w_std=0.3)
    y = torch.arange(n_tok, dtype=torch.int32, device=cuda) * 2 + 1
    y[0] = 0
    y[1] = vocab - 1
    y[2:258] = torch.arange(768, 1024, dtype=torch.int32, device=cuda)
    y = y.clamp_(max=vocab - 1)
    _parity(H, W, y, label="every tile position")


def test_extreme_logits(cuda):
    """Large logits: one dominant entry per row, and rows far from zero."""
    import torch

    vocab, d, n = 700, 64, 40
    H = torch.zeros(n, d, dtype=torch.float32)
    W = torch.zeros(vocab, d, dtype=torch.float32)
    W[5, 0] = 60.0
    W[:, 1] = 1.0
    H[:, 0] = 1.0
    H[:, 1] = torch.linspace(-300, 300, n)  # shifts every logit of a row
    y = torch.full((n,), 5, dtype=torch.int32)
    y[::2] = 6
    _parity(H.to(cuda), W.to(cuda), y.to(cuda), label="extreme")


def test_row_position_invariance(cuda):
    """One hidden state placed at every row of a 256-token block, and alone."""
    import torch

    vocab, d = 3000, 256
    H, W, y = _random_head(256, d, vocab, torch.bfloat16, seed=11, device=cuda, w_std=0.05)
    itl = _itl()
    probe = H[17].clone()
    tok = y[17].clone()
    alone_lp, alone_lse = itl.lmhead_logprob(probe[None].contiguous(), W, tok[None].contiguous())
    for pos in range(256):
        Hp = H.clone()
        yp = y.clone()
        Hp[pos] = probe
        yp[pos] = tok
        lp, lse = itl.lmhead_logprob(Hp, W, yp)
        assert same_bits(lp[pos:pos + 1], alone_lp) and same_bits(lse[pos:pos + 1], alone_lse), pos


@pytest.mark.parametrize(
    "d,vocab,dtype_name",
    [
        (2560, 151936, "bf16"),   # 256 slices of 2 or 3 tiles, partial last tile
        (7168, 129280, "bf16"),   # 112 K steps: the wide kernel stages the token block two steps ahead
        (128, 4096 + 37, "bf16"),  # one tile per slice, last tile of 37 rows
        (64, 1000, "f32"),        # fp32 MFMA
    ],
)
def test_narrow_and_wide_kernels_agree(cuda, d, vocab, dtype_name):
    """Calls of at most narrow_max_tokens tokens (build info) run the narrow
    kernel on 64-token blocks, calls of up to narrow128_max_tokens on one
    128-token block, larger ones the 256-token block kernel: the same tokens
    give the same bits either way, at every row of a narrow block and across
    blocks."""
    import re
    import torch

    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    H, W, y = _random_head(600, d, vocab, dt, seed=d + vocab, device=cuda)
    itl = _itl()
    limit = int(re.search(r"narrow_max_tokens=(\d+)", itl.build_info()).group(1))
    limit128 = int(re.search(r"narrow128_max_tokens=(\d+)", itl.build_info()).group(1))
    assert 1 <= limit < limit128
    lp, lse = itl.lmhead_logprob(H, W, y)  # wide kernel
    for lo, n in ((0, 1), (5, 7), (100, min(limit, 33)), (300, limit), (472, limit + 1), (200, 100),
                  (210, limit128), (200, limit128 + 1)):
        lp_n, lse_n = itl.lmhead_logprob(H[lo:lo + n], W, y[lo:lo + n])
        assert same_bits(lp_n, lp[lo:lo + n]) and same_bits(lse_n, lse[lo:lo + n]), (lo, n)
    # a narrow call at every row position of the 64-token block, and of the
    # 128-token one
    probe_lp = lp[17:18]
    for size in (min(limit, 64), limit128):
        for pos in range(size):
            Hp = H[:size].clone()
            yp = y[:size].clone()
            Hp[pos] = H[17]
            yp[pos] = y[17]
            lp_p, _ = itl.lmhead_logprob(Hp, W, yp)
            assert same_bits(lp_p[pos:pos + 1], probe_lp), (size, pos)


def test_run_to_run_determinism(cuda):
    import torch

    H, W, y = _random_head(1000, 512, 20000, torch.bfloat16, seed=3, device=cuda)
    itl = _itl()
    a = itl.lmhead_logprob(H, W, y)
    for _ in range(3):
        b = itl.lmhead_logprob(H, W, y)
        assert same_bits(a[0], b[0]) and same_bits(a[1], b[1])


def test_lse_optional_and_empty(cuda):
    import torch

    itl = _itl()
    H, W, y = _random_head(10, 64, 500, torch.bfloat16, seed=5, device=cuda)
    lp, lse = itl.lmhead_logprob(H, W, y, want_lse=False)
    assert lse is None
    lp2, _ = itl.lmhead_logprob(H, W, y)
    assert same_bits(lp, lp2)
    e = torch.empty(0, 64, dtype=torch.bfloat16, device=cuda)
    lp0, _ = itl.lmhead_logprob(e, W, torch.empty(0, dtype=torch.int32, device=cuda))
    assert lp0.numel() == 0


def test_check_inputs_flags_bad_tokens(cuda):
    import torch

    itl = _itl()
    y = torch.tensor([0, 5, 9], dtype=torch.int32, device=cuda)
    itl.check_inputs(y, 10)
    with pytest.raises(itl.ItlError):
        itl.check_inputs(y, 9)
    off = torch.tensor([0, 2, 2, 3], dtype=torch.int64, device=cuda)
    with pytest.raises(itl.ItlError):
        itl.check_inputs(y, 10, off)
    itl.check_inputs(y, 10, torch.tensor([0, 2, 3], dtype=torch.int64, device=cuda))


@pytest.mark.parametrize("key", ["qwen2.5-1.5b-head", "qwen3-4b-head", "large-moe-head"])
def test_full_size_head_sampled_parity(cuda, key):
    """Full-size heads in the benchmark's launch configuration; the oracle
    recomputes a seeded sample of 48 tokens one by one."""
    import torch
    import oracle
    from synth import WORKLOADS, draw_head, draw_layout, sample_tokens, token_subset

    wl = WORKLOADS[key]
    lay = draw_layout(wl)
    say(f"[{key}] n_tok={lay.n_tok} d={wl.d} V={wl.vocab}")
    H, W = draw_head(wl, lay.n_tok, device=cuda)
    y = sample_tokens(H, W, wl)
    itl = _itl()
    lp, lse = itl.lmhead_logprob(H, W, y)
    torch.cuda.synchronize()
    assert bool(torch.all(lp <= 0)) and bool(torch.all(torch.isfinite(lp)))
    idx = token_subset(lay.n_tok, 48, seed=wl.index)
    idx_t = torch.from_numpy(idx).to(cuda)
    Hs = H.index_select(0, idx_t)
    lp_o, lse_o = oracle.lmhead_logprob(host_array(Hs), host_array(W), y.index_select(0, idx_t).cpu().numpy())
    e_lp = float(np.max(np.abs(lp.index_select(0, idx_t).cpu().numpy() - lp_o)))
    e_lse = float(np.max(np.abs(lse.index_select(0, idx_t).cpu().numpy() - lse_o)))
    say(f"[{key}] sampled max|dlp|={e_lp:.3e} max|dlse|={e_lse:.3e}")
    assert e_lp <= TOL_LP and e_lse <= TOL_LP
    lp2, _ = itl.lmhead_logprob(H, W, y, want_lse=False)
    assert same_bits(lp, lp2)
