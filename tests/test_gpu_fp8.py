"""GPU parity of the FP8 (E4M3) head: itl_quantize_rows_fp8 bit for bit
against the oracle's quantisation (codes and scales are integer decisions
taken in float32 on both sides), and itl_lmhead_logprob_fp8 within 1e-3 of
the float64 oracle on the oracle's own codes. Small cases compare every
token; the qwen3-4b head at full size compares all of W's codes and a seeded
sample of tokens. Batch and position invariance and run-to-run bits too."""

import numpy as np
import pytest

from helpers import same_bits, say

pytestmark = pytest.mark.gpu

TOL_LP = 1e-3


def _itl():
    import invariant_token_logprobs_lm_amd as itl

    return itl


def _host_f32(X):
    import torch

    return X.float().cpu().numpy()


@pytest.mark.parametrize("n,d,dtype_name,scale_pow", [
    (37, 128, "bf16", 0), (200, 256, "f32", 0), (64, 2560, "bf16", 0),
    (50, 384, "f32", -30),   # tiny values: scales far below 1, many subnormal codes
    (50, 128, "f32", 20),    # large values
    (9, 8192, "bf16", 0),    # rows too long to keep in registers: the two-pass path
    (9, 4096, "f32", 0),
])
def test_quantize_rows_bit_exact(cuda, n, d, dtype_name, scale_pow):
    import torch
    from oracle import fp8

    g = torch.Generator(device="cpu").manual_seed(n * 31 + d)
    X = torch.randn(n, d, generator=g) * (2.0 ** scale_pow)
    X[3] = 0.0                     # an all-zero row
    X[5, ::7] = 0.0
    X[6] = X[6] * 1e-3             # a row with a different range
    X[7, 1] = -X[7].abs().max() * 2  # a negative maximum
    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    X = X.to(dt)
    itl = _itl()
    Xq, s = itl.quantize_rows_fp8(X.to(cuda))
    q_o, s_o = fp8.quantize_rows_fp8(_host_f32(X))
    assert np.array_equal(Xq.cpu().numpy(), q_o)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_o.view(np.uint32))
    say(f"[fp8 quantize] {n}x{d} {dtype_name} 2^{scale_pow}: codes and scales bit-identical")


@pytest.mark.gpu
@pytest.mark.parametrize("dtype_name", ["bf16", "f32"])
def test_quantize_rows_unaligned_input(cuda, dtype_name):
    """X whose base is not 16-byte aligned takes the two-pass path; the codes
    are the same."""
    import torch
    from oracle import fp8

    n, d = 9, 256
    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    g = torch.Generator(device="cpu").manual_seed(77)
    X = (torch.randn(n, d, generator=g) * 3.0).to(dt)
    buf = torch.zeros(n * d + 8, dtype=dt, device=cuda)
    buf[1:1 + n * d] = X.reshape(-1).to(cuda)
    Xv = buf[1:1 + n * d].view(n, d)
    assert Xv.data_ptr() % 16 != 0
    itl = _itl()
    Xq, s = itl.quantize_rows_fp8(Xv)
    q_o, s_o = fp8.quantize_rows_fp8(_host_f32(X))
    assert np.array_equal(Xq.cpu().numpy(), q_o)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_o.view(np.uint32))


def _oracle_quantized_head(n_tok, d, vocab, seed, w_std=0.05):
    import torch
    from oracle import fp8

    g = torch.Generator(device="cpu").manual_seed(seed)
    H = torch.randn(n_tok, d, generator=g).to(torch.bfloat16)
    W = (torch.randn(vocab, d, generator=g) * w_std).to(torch.bfloat16)
    y = torch.randint(0, vocab, (n_tok,), generator=g, dtype=torch.int32)
    Hq, hs = fp8.quantize_rows_fp8(_host_f32(H))
    Wq, ws = fp8.quantize_rows_fp8(_host_f32(W))
    return Hq, hs, Wq, ws, y.numpy()


def _to_dev(cuda, *arrays):
    import torch

    return [torch.from_numpy(np.ascontiguousarray(a)).to(cuda) for a in arrays]


@pytest.mark.parametrize("n_tok,d,vocab", [
    (700, 256, 5000),          # 3 token blocks (ragged), 20 tiles
    (300, 128, 4096 + 37),     # one K step per tile (wide kernel, 2 token blocks); last tile of 37 rows
    (1, 128, 300),             # one token (narrow kernel)
    (64, 256, 3000),           # a full narrow block
    (513, 384, 8192 + 256),    # d = 3 K steps
    (5200, 128, 150 * 256 - 17),  # d = 128 with many tokens: the wide kernel, 21 token blocks
    (3400, 256, 150 * 256 - 17),  # 14 x 150 > 2048: several slices per workgroup (wide kernel)
    (100, 256, 200),           # one partial vocabulary tile, one slice (narrow kernel, one 128-token block)
    (65, 128, 1000),           # the fewest tokens of the 128-token narrow block
    (128, 384, 3000),          # a full 128-token narrow block
    (129, 128, 1000),          # the fewest tokens the wide kernel takes
])
def test_lmhead_fp8_parity(cuda, n_tok, d, vocab):
    from oracle import fp8

    Hq, hs, Wq, ws, y = _oracle_quantized_head(n_tok, d, vocab, seed=n_tok + vocab)
    lp_o, lse_o = fp8.lmhead_logprob_fp8(Hq, hs, Wq, ws, y)
    itl = _itl()
    Hq_d, hs_d, Wq_d, ws_d, y_d = _to_dev(cuda, Hq, hs, Wq, ws, y)
    lp, lse = itl.lmhead_logprob_fp8(Hq_d, hs_d, Wq_d, ws_d, y_d)
    e_lp = float(np.max(np.abs(lp.cpu().numpy() - lp_o)))
    e_lse = float(np.max(np.abs(lse.cpu().numpy() - lse_o)))
    say(f"[fp8 parity {n_tok}x{d}x{vocab}] max|dlp|={e_lp:.3e} max|dlse|={e_lse:.3e}")
    assert e_lp <= TOL_LP and e_lse <= TOL_LP
    assert float(lp.max()) <= 0.0


def test_lmhead_fp8_many_tiles_per_slice(cuda):
    """A vocabulary of 1,290 tiles (5-6 per slice of 256): the narrow kernel
    fetches its row scales four tiles at a time, so a slice takes two
    groups. The logprobs match the oracle, and a token has the same bits in
    a narrow call (3 tokens) as in a wide one (70)."""
    from oracle import fp8

    vocab = 1290 * 256 - 101
    Hq, hs, Wq, ws, y = _oracle_quantized_head(70, 128, vocab, seed=41)
    y[:3] = [vocab - 1, 4 * 256 * 256 + 5, 17]  # sampled rows in the last tile, a high one, the first
    itl = _itl()
    Hq_d, hs_d, Wq_d, ws_d, y_d = _to_dev(cuda, Hq, hs, Wq, ws, y)
    lp_n, lse_n = itl.lmhead_logprob_fp8(Hq_d[:3], hs_d[:3], Wq_d, ws_d, y_d[:3])
    lp_o, lse_o = fp8.lmhead_logprob_fp8(Hq[:3], hs[:3], Wq, ws, y[:3])
    e_lp = float(np.max(np.abs(lp_n.cpu().numpy() - lp_o)))
    e_lse = float(np.max(np.abs(lse_n.cpu().numpy() - lse_o)))
    say(f"[fp8 many tiles per slice] max|dlp|={e_lp:.3e} max|dlse|={e_lse:.3e}")
    assert e_lp <= TOL_LP and e_lse <= TOL_LP
    lp_w, lse_w = itl.lmhead_logprob_fp8(Hq_d, hs_d, Wq_d, ws_d, y_d)
    assert same_bits(lp_w[:3], lp_n) and same_bits(lse_w[:3], lse_n)


@pytest.mark.parametrize("d", [256, 128, 6272])  # 6272: 49 K steps, the token block staged two steps ahead
def test_lmhead_fp8_invariance(cuda, d):
    """The same token gives the same bits alone, at every row of a block, in
    any sub-batch (wide and narrow kernels); and run to run."""
    import torch

    Hq, hs, Wq, ws, y = _oracle_quantized_head(600, d, 3000, seed=5)
    itl = _itl()
    Hq_d, hs_d, Wq_d, ws_d, y_d = _to_dev(cuda, Hq, hs, Wq, ws, y)
    lp, lse = itl.lmhead_logprob_fp8(Hq_d, hs_d, Wq_d, ws_d, y_d)
    for lo, n in ((0, 1), (17, 5), (100, 64), (150, 65), (200, 128), (330, 129), (300, 257)):
        a, b = itl.lmhead_logprob_fp8(Hq_d[lo:lo + n], hs_d[lo:lo + n], Wq_d, ws_d, y_d[lo:lo + n])
        assert same_bits(a, lp[lo:lo + n]) and same_bits(b, lse[lo:lo + n]), (lo, n)
    for pos in (0, 1, 31, 32, 127, 128, 200, 255):
        Hp, hp, yp = Hq_d[:256].clone(), hs_d[:256].clone(), y_d[:256].clone()
        Hp[pos], hp[pos], yp[pos] = Hq_d[17], hs_d[17], y_d[17]
        a, _ = itl.lmhead_logprob_fp8(Hp, hp, Wq_d, ws_d, yp)
        assert same_bits(a[pos:pos + 1], lp[17:18]), pos
    # narrow kernel: every row of a 64-token block (calls of at most 64
    # tokens) and of the 128-token block (calls of 65 to 128)
    for size in (64, 128):
        for pos in range(size):
            Hp, hp, yp = Hq_d[:size].clone(), hs_d[:size].clone(), y_d[:size].clone()
            Hp[pos], hp[pos], yp[pos] = Hq_d[17], hs_d[17], y_d[17]
            a, _ = itl.lmhead_logprob_fp8(Hp, hp, Wq_d, ws_d, yp)
            assert same_bits(a[pos:pos + 1], lp[17:18]), ("narrow", size, pos)
    again = itl.lmhead_logprob_fp8(Hq_d, hs_d, Wq_d, ws_d, y_d)
    torch.cuda.synchronize()
    assert same_bits(again[0], lp) and same_bits(again[1], lse)


def test_lmhead_fp8_full_size_head(cuda):
    """The qwen3-4b head at full size: the GPU's W codes equal the oracle's
    for every row; sampled tokens' logprobs (their H rows quantised by the
    oracle too, and checked equal to the GPU's codes) within 1e-3."""
    import torch
    from oracle import fp8
    from synth import WORKLOADS, draw_head, draw_layout, sample_tokens, token_subset

    wl = WORKLOADS["qwen3-4b-head"]
    lay = draw_layout(wl)
    H, W = draw_head(wl, lay.n_tok, device=cuda)
    y = sample_tokens(H, W, wl)
    itl = _itl()
    Wq, ws = itl.quantize_rows_fp8(W)
    Hq, hs = itl.quantize_rows_fp8(H)
    lp, lse = itl.lmhead_logprob_fp8(Hq, hs, Wq, ws, y)
    Wq_h, ws_h = Wq.cpu().numpy(), ws.cpu().numpy()
    Wf = W.float().cpu().numpy()
    for r0 in range(0, wl.vocab, 16384):
        q_o, s_o = fp8.quantize_rows_fp8(Wf[r0:r0 + 16384])
        assert np.array_equal(Wq_h[r0:r0 + 16384], q_o), r0
        assert np.array_equal(ws_h[r0:r0 + 16384].view(np.uint32), s_o.view(np.uint32)), r0
    del Wf
    tok = token_subset(lay.n_tok, 32, seed=11)
    Hs = H.index_select(0, torch.from_numpy(tok).to(cuda)).float().cpu().numpy()
    hq_o, hs_o = fp8.quantize_rows_fp8(Hs)
    assert np.array_equal(Hq.cpu().numpy()[tok], hq_o)
    assert np.array_equal(hs.cpu().numpy()[tok].view(np.uint32), hs_o.view(np.uint32))
    lp_o, lse_o = fp8.lmhead_logprob_fp8(hq_o, hs_o, Wq_h, ws_h, y.cpu().numpy()[tok])
    e_lp = float(np.max(np.abs(lp.cpu().numpy()[tok] - lp_o)))
    say(f"[fp8 qwen3-4b-head] n_tok={lay.n_tok}: W codes bit-identical; sampled max|dlp|={e_lp:.3e}")
    assert e_lp <= TOL_LP
    assert float(lp.max()) <= 0.0


# ---- MXFP4 weights ----

@pytest.mark.parametrize("n,d,dtype_name,scale_pow", [
    (37, 128, "bf16", 0), (64, 2560, "bf16", 0), (50, 384, "f32", -128),  # subnormal-range values
    (50, 256, "f32", 100), (20, 128, "f32", -3)])
def test_quantize_mxfp4_bit_exact(cuda, n, d, dtype_name, scale_pow):
    import torch
    from oracle import fp8

    g = torch.Generator(device="cpu").manual_seed(n * 13 + d)
    X = torch.randn(n, d, generator=g, dtype=torch.float64) * (2.0 ** scale_pow)
    X[2] = 0.0
    X[4, :32] = 0.0                 # one all-zero block
    X[5, 32:64] = X[5, 32:64] * 1e-6
    X = X.float()
    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    X = X.to(dt)
    itl = _itl()
    q, s = itl.quantize_rows_mxfp4(X.to(cuda))
    q_o, s_o = fp8.quantize_rows_mxfp4(_host_f32(X))
    assert np.array_equal(s.cpu().numpy(), s_o)
    assert np.array_equal(q.cpu().numpy(), q_o)
    say(f"[mxfp4 quantize] {n}x{d} {dtype_name} 2^{scale_pow}: codes and scales bit-identical")


def _oracle_mxfp4_head(n_tok, d, vocab, seed, w_std=0.05):
    import torch
    from oracle import fp8

    g = torch.Generator(device="cpu").manual_seed(seed)
    H = torch.randn(n_tok, d, generator=g).to(torch.bfloat16)
    W = (torch.randn(vocab, d, generator=g) * w_std).to(torch.bfloat16)
    y = torch.randint(0, vocab, (n_tok,), generator=g, dtype=torch.int32)
    Hq, hs = fp8.quantize_rows_fp8(_host_f32(H))
    Wq, ws = fp8.quantize_rows_mxfp4(_host_f32(W))
    return Hq, hs, Wq, ws, y.numpy()


@pytest.mark.parametrize("n_tok,d,vocab", [
    (700, 256, 5000), (300, 128, 4096 + 37), (1, 128, 300), (64, 256, 3000), (513, 384, 8192 + 256),
    (5200, 128, 150 * 256 - 17),
    (65, 128, 1000), (100, 256, 200), (128, 384, 3000),  # the 128-token narrow block
    (129, 128, 1000)])                                   # the fewest tokens of the wide kernel
def test_lmhead_mxfp4_parity(cuda, n_tok, d, vocab):
    from oracle import fp8

    Hq, hs, Wq, ws, y = _oracle_mxfp4_head(n_tok, d, vocab, seed=2 * n_tok + vocab)
    lp_o, lse_o = fp8.lmhead_logprob_mxfp4(Hq, hs, Wq, ws, y)
    itl = _itl()
    Hq_d, hs_d, Wq_d, ws_d, y_d = _to_dev(cuda, Hq, hs, Wq, ws, y)
    lp, lse = itl.lmhead_logprob_mxfp4(Hq_d, hs_d, Wq_d, ws_d, y_d)
    e_lp = float(np.max(np.abs(lp.cpu().numpy() - lp_o)))
    e_lse = float(np.max(np.abs(lse.cpu().numpy() - lse_o)))
    say(f"[mxfp4 parity {n_tok}x{d}x{vocab}] max|dlp|={e_lp:.3e} max|dlse|={e_lse:.3e}")
    assert e_lp <= TOL_LP and e_lse <= TOL_LP
    assert float(lp.max()) <= 0.0


def test_lmhead_mxfp4_invariance(cuda):
    import torch

    Hq, hs, Wq, ws, y = _oracle_mxfp4_head(600, 256, 3000, seed=9)
    itl = _itl()
    Hq_d, hs_d, Wq_d, ws_d, y_d = _to_dev(cuda, Hq, hs, Wq, ws, y)
    lp, lse = itl.lmhead_logprob_mxfp4(Hq_d, hs_d, Wq_d, ws_d, y_d)
    for lo, n in ((0, 1), (17, 5), (100, 64), (150, 65), (200, 128), (330, 129), (300, 257)):
        a, b = itl.lmhead_logprob_mxfp4(Hq_d[lo:lo + n], hs_d[lo:lo + n], Wq_d, ws_d, y_d[lo:lo + n])
        assert same_bits(a, lp[lo:lo + n]) and same_bits(b, lse[lo:lo + n]), (lo, n)
    for pos in (0, 31, 32, 128, 255):
        Hp, hp, yp = Hq_d[:256].clone(), hs_d[:256].clone(), y_d[:256].clone()
        Hp[pos], hp[pos], yp[pos] = Hq_d[17], hs_d[17], y_d[17]
        a, _ = itl.lmhead_logprob_mxfp4(Hp, hp, Wq_d, ws_d, yp)
        assert same_bits(a[pos:pos + 1], lp[17:18]), pos
    # narrow kernel: every row of a 64-token block (calls of at most 64
    # tokens) and of the 128-token block (calls of 65 to 128)
    for size in (64, 128):
        for pos in range(size):
            Hp, hp, yp = Hq_d[:size].clone(), hs_d[:size].clone(), y_d[:size].clone()
            Hp[pos], hp[pos], yp[pos] = Hq_d[17], hs_d[17], y_d[17]
            a, _ = itl.lmhead_logprob_mxfp4(Hp, hp, Wq_d, ws_d, yp)
            assert same_bits(a[pos:pos + 1], lp[17:18]), ("narrow", size, pos)
    again = itl.lmhead_logprob_mxfp4(Hq_d, hs_d, Wq_d, ws_d, y_d)
    torch.cuda.synchronize()
    assert same_bits(again[0], lp) and same_bits(again[1], lse)


def test_lmhead_mxfp4_full_size_head(cuda):
    """The qwen3-4b head at full size with MXFP4 weights: every W code and
    scale equal to the oracle's; sampled tokens within 1e-3."""
    import torch
    from oracle import fp8
    from synth import WORKLOADS, draw_head, draw_layout, sample_tokens, token_subset

    wl = WORKLOADS["qwen3-4b-head"]
    lay = draw_layout(wl)
    H, W = draw_head(wl, lay.n_tok, device=cuda)
    y = sample_tokens(H, W, wl)
    itl = _itl()
    Wq, ws = itl.quantize_rows_mxfp4(W)
    Hq, hs = itl.quantize_rows_fp8(H)
    lp, lse = itl.lmhead_logprob_mxfp4(Hq, hs, Wq, ws, y)
    Wq_h, ws_h = Wq.cpu().numpy(), ws.cpu().numpy()
    Wf = W.float().cpu().numpy()
    for r0 in range(0, wl.vocab, 16384):
        q_o, s_o = fp8.quantize_rows_mxfp4(Wf[r0:r0 + 16384])
        assert np.array_equal(Wq_h[r0:r0 + 16384], q_o) and np.array_equal(ws_h[r0:r0 + 16384], s_o), r0
    del Wf
    tok = token_subset(lay.n_tok, 32, seed=12)
    Hs = H.index_select(0, torch.from_numpy(tok).to(cuda)).float().cpu().numpy()
    hq_o, hs_o = fp8.quantize_rows_fp8(Hs)
    assert np.array_equal(Hq.cpu().numpy()[tok], hq_o)
    lp_o, _ = fp8.lmhead_logprob_mxfp4(hq_o, hs_o, Wq_h, ws_h, y.cpu().numpy()[tok])
    e_lp = float(np.max(np.abs(lp.cpu().numpy()[tok] - lp_o)))
    say(f"[mxfp4 qwen3-4b-head] n_tok={lay.n_tok}: W codes bit-identical; sampled max|dlp|={e_lp:.3e}")
    assert e_lp <= TOL_LP
    assert float(lp.max()) <= 0.0


@pytest.mark.gpu
def test_quantized_heads_empty_calls(cuda):
    """Zero rows and zero tokens are no-ops that return empty results."""
    import torch

    itl = _itl()
    d, vocab = 256, 3000
    W = (torch.randn(vocab, d, generator=torch.Generator(device="cpu").manual_seed(3)) * 0.05).to(torch.bfloat16)
    W = W.to(cuda)
    Wq, ws = itl.quantize_rows_fp8(W)
    W4, s4 = itl.quantize_rows_mxfp4(W)
    H0 = torch.empty(0, d, dtype=torch.bfloat16, device=cuda)
    Hq0, hs0 = itl.quantize_rows_fp8(H0)
    assert Hq0.shape == (0, d) and hs0.shape == (0,)
    W40, s40 = itl.quantize_rows_mxfp4(H0)
    assert W40.shape == (0, d // 2) and s40.shape == (0, d // 32)
    y0 = torch.empty(0, dtype=torch.int32, device=cuda)
    lp, lse = itl.lmhead_logprob_fp8(Hq0, hs0, Wq, ws, y0)
    assert lp.shape == (0,) and lse.shape == (0,)
    lp, lse = itl.lmhead_logprob_mxfp4(Hq0, hs0, W4, s4, y0)
    assert lp.shape == (0,) and lse.shape == (0,)
    torch.cuda.synchronize()
