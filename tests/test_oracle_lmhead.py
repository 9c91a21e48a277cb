"""Pins for the oracle's logits, log-softmax and sampled-token logprob.

Each test checks the oracle against something other than itself: exact
rational arithmetic, 60-digit decimal arithmetic, closed forms, invariants,
and torch's own float64 log_softmax (a library routine the oracle does not
use).
"""

import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _bf16_bits(x):
    """Round float32 values to bfloat16 (nearest even) and return the bits."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def test_bf16_decode_known_patterns():
    # IEEE binary32 upper halves: sign | 8-bit exponent | 7 mantissa bits.
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x4049], dtype=np.uint16)
    got = oracle.to_f64(bits)
    want = [1.0, -2.0, 1.0 + 2.0**-7, 2.0**-133, math.inf, -math.inf, 0.0, -0.0, 3.140625]
    for g, w in zip(got, want):
        assert g == w
    assert math.copysign(1.0, got[7]) == -1.0


def test_logits_equal_exact_rational_dot_products():
    rng = np.random.default_rng(11)
    for d in (64, 2560):
        H = _bf16_bits(rng.normal(0, 1, (3, d)))
        W = _bf16_bits(rng.normal(0, 0.02, (5, d)))
        z = oracle.logits(H, W)
        Hf = oracle.to_f64(H)
        Wf = oracle.to_f64(W)
        for t in range(3):
            for v in range(5):
                exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(Hf[t], Wf[v]))
                mag = float(np.abs(Hf[t] * Wf[v]).sum())
                assert abs(z[t, v] - float(exact)) <= d * 2.0**-52 * mag + 1e-300


def _decimal_logprob(zrow, y):
    getcontext().prec = 60
    zs = [Decimal(Fraction(float(v)).numerator) / Decimal(Fraction(float(v)).denominator) for v in zrow]
    total = sum((x.exp() for x in zs), Decimal(0))
    return zs[y] - total.ln()


@pytest.mark.parametrize("V", [2, 7, 33, 64])
def test_logprob_matches_60_digit_bruteforce(V):
    rng = np.random.default_rng(V)
    d = 8
    H = rng.normal(0, 1.5, (4, d)).astype(np.float32)
    W = rng.normal(0, 1.0, (V, d)).astype(np.float32)
    y = rng.integers(0, V, 4)
    lp, lse = oracle.lmhead_logprob(H, W, y)
    # exact logits as rationals, then the unshifted definition in 60 digits
    for t in range(4):
        zrow = [
            float(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(H[t], W[v])))
            for v in range(V)
        ]
        want = _decimal_logprob(zrow, int(y[t]))
        assert abs(lp[t] - float(want)) <= 1e-12
        assert abs((lp[t] + lse[t]) - zrow[int(y[t])]) <= 1e-12


def test_uniform_logits_give_minus_log_vocab_exactly():
    V, d = 1000, 16
    y = np.array([0, 17, 999])
    lp, lse = oracle.lmhead_logprob(np.zeros((3, d), np.float32), np.ones((V, d), np.float32), y)
    assert np.all(lp == -math.log(V))
    W = np.tile(np.linspace(-1, 1, d, dtype=np.float32), (V, 1))
    H = np.random.default_rng(0).normal(0, 1, (3, d)).astype(np.float32)
    lp, lse = oracle.lmhead_logprob(H, W, y)
    # every logit of a row is the same number m, so lp = m - (m + log V):
    # equal to -log V up to the rounding of m + log V
    m = lse - math.log(V)
    assert np.all(np.abs(lp + math.log(V)) <= 2.0**-51 * (np.abs(m) + math.log(V)))


def test_one_dominant_logit():
    V = 50
    W = np.zeros((V, 1), np.float32)
    W[3, 0] = 10.0
    H = np.ones((2, 1), np.float32)
    lp, _ = oracle.lmhead_logprob(H, W, np.array([3, 4]))
    # p(3) = e^10 / (e^10 + 49), p(4) = 1 / (e^10 + 49)
    assert abs(lp[0] - (-math.log1p(49 * math.exp(-10.0)))) <= 1e-15
    assert abs(lp[1] - (-10.0 - math.log1p(49 * math.exp(-10.0)))) <= 1e-13
    W[3, 0] = 100.0
    lp, _ = oracle.lmhead_logprob(H, W, np.array([3, 4]))
    assert -1e-40 <= lp[0] <= 0.0
    assert abs(lp[1] - (-100.0)) <= 1e-12


def test_shift_invariance():
    rng = np.random.default_rng(5)
    n, d, V = 6, 32, 300
    H = rng.normal(0, 1, (n, d))
    W = rng.normal(0, 0.3, (V, d))
    y = rng.integers(0, V, n)
    lp0, lse0 = oracle.lmhead_logprob(H, W, y)
    # A constant column in W (all ones) times a per-token value adds that
    # value to every logit of the token; the logprob must not move.
    shift = rng.normal(0, 20, (n, 1))
    lp1, lse1 = oracle.lmhead_logprob(np.hstack([H, shift]), np.hstack([W, np.ones((V, 1))]), y)
    assert np.max(np.abs(lp1 - lp0)) <= 1e-11
    assert np.max(np.abs((lse1 - lse0) - shift[:, 0])) <= 1e-11


def test_logprob_nonpositive_and_softmax_sums_to_one():
    rng = np.random.default_rng(9)
    d, V = 64, 4096
    H = _bf16_bits(rng.normal(0, 1, (1, d)))
    W = _bf16_bits(rng.normal(0, 0.5, (V, d)))
    y_all = np.arange(V)
    lp, _ = oracle.lmhead_logprob(np.repeat(H, V, axis=0), W, y_all)
    assert np.all(lp <= 0)
    assert abs(math.fsum(np.exp(lp)) - 1.0) <= 1e-12


def test_matches_torch_float64_log_softmax():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    n, d, V = 40, 128, 1024
    H = rng.normal(0, 1, (n, d)).astype(np.float32)
    W = rng.normal(0, 0.05, (V, d)).astype(np.float32)
    y = rng.integers(0, V, n)
    lp, lse = oracle.lmhead_logprob(H, W, y, token_block=16, vocab_chunk=100)
    z = torch.from_numpy(H).double() @ torch.from_numpy(W).double().T
    ref = torch.log_softmax(z, dim=1)[torch.arange(n), torch.from_numpy(y)]
    assert np.max(np.abs(lp - ref.numpy())) <= 1e-12
    assert np.max(np.abs(lse - torch.logsumexp(z, dim=1).numpy())) <= 1e-12


def test_rejects_out_of_range_tokens():
    with pytest.raises(ValueError):
        oracle.lmhead_logprob(np.zeros((2, 4), np.float32), np.zeros((8, 4), np.float32), np.array([0, 8]))
    with pytest.raises(ValueError):
        oracle.lmhead_logprob(np.zeros((2, 4), np.float32), np.zeros((8, 4), np.float32), np.array([-1, 0]))


def test_empty_and_nan_propagation():
    lp, lse = oracle.lmhead_logprob(np.zeros((0, 4), np.float32), np.zeros((8, 4), np.float32), np.zeros(0, np.int64))
    assert lp.shape == (0,) and lse.shape == (0,)
    H = np.zeros((1, 4), np.float32)
    H[0, 1] = np.nan
    lp, _ = oracle.lmhead_logprob(H, np.ones((8, 4), np.float32), np.array([2]))
    assert np.isnan(lp[0])
