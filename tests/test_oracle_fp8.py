"""Pins of the FP8 (E4M3) oracle (oracle/fp8.py): the code table against the
format's definition, hand-picked roundings, per-row scales, and the fp8
logprob against the (independently pinned) bf16 head oracle."""

import math

import numpy as np
import pytest

import oracle
from oracle import fp8


def _value_by_definition(c):
    """E4M3 value of code c from the bit fields, written out directly."""
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 7
    if e == 0xF and m == 7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1 + m / 8) * 2.0 ** (e - 7)


def test_decode_matches_the_bit_fields():
    codes = np.arange(256, dtype=np.uint8)
    got = fp8.e4m3_decode(codes)
    for c in range(256):
        w = _value_by_definition(c)
        assert (math.isnan(w) and math.isnan(got[c])) or got[c] == w, c
    finite = got[~np.isnan(got)]
    assert finite.max() == 448.0 and finite.min() == -448.0
    assert np.min(np.abs(finite[finite != 0])) == 2.0 ** -9


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = fp8.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(fp8.e4m3_encode(vals), codes)


@pytest.mark.parametrize("x,code", [
    (1.0, 0x38), (-1.0, 0xB8), (448.0, 0x7E), (-448.0, 0xFE), (2.0 ** -9, 0x01), (2.0 ** -6, 0x08),
    (0.0, 0x00), (-0.0, 0x80),
    (0.5 * 2.0 ** -9, 0x00),      # tie between 0 and 2^-9: even code 0
    (1.5 * 2.0 ** -9, 0x02),      # tie between 1 and 2 (x 2^-9): even code 2
    (2.5 * 2.0 ** -9, 0x02),      # tie between 2 and 3: even 2
    (1.0625, 0x38),               # tie between 1 and 1.125: even mantissa 0
    (1.1875, 0x3A),               # tie between 1.125 and 1.25: even mantissa 2
    (7.99 * 2.0 ** -9, 0x08),     # rounds up into the smallest normal
    (15.9, 0x58),                 # rounds to 16 = 2^4: exponent carry
    (460.0, 0x7E), (464.0, 0x7E), (470.0, 0x7E), (1e6, 0x7E), (-1e6, 0xFE),  # saturate at 448
])
def test_hand_picked_roundings(x, code):
    assert int(fp8.e4m3_encode(np.float32(x))) == code


def test_row_scales_and_zero_row():
    X = np.array([[1.0, -2.0, 0.5, 0.0], [0.0, 0.0, 0.0, 0.0], [448.0, 1.0, -448.0, 3.5]], dtype=np.float32)
    q, s = fp8.quantize_rows_fp8(X)
    assert s.dtype == np.float32
    assert s[0] == np.float32(2.0) / np.float32(448.0) and s[1] == 1.0 and s[2] == 1.0
    assert np.all(q[1] == 0)
    # the row maximum maps to +-448 (codes 0x7E / 0xFE)
    assert q[0, 1] == 0xFE and q[2, 0] == 0x7E and q[2, 2] == 0xFE
    # values representable after scaling come back exactly
    assert fp8.e4m3_decode(q[2, 3]) == 3.5 and fp8.e4m3_decode(q[2, 1]) == 1.0
    # dequantised values stay within half a code step (relative 1/16) of the input
    rng = np.random.default_rng(0)
    Y = rng.standard_normal((50, 256)).astype(np.float32)
    qy, sy = fp8.quantize_rows_fp8(Y)
    back = fp8.e4m3_decode(qy) * sy[:, None]
    big = np.abs(Y) >= 2.0 ** -6 * sy[:, None]
    assert np.all(np.abs(back - Y)[big] <= np.abs(Y)[big] / 16 * (1 + 1e-6))
    assert np.all(np.abs(back - Y)[~big] <= 2.0 ** -10 * sy[:, None].repeat(256, 1)[~big] * (1 + 1e-6))


def test_fp8_logprob_exact_tiny_head():
    """Codes whose values are small integers: z is an exact integer dot
    product; compare with the closed-form log-softmax."""
    Hq = fp8.e4m3_encode(np.array([[1, 2, 0, -1], [0, 0, 3, 1]], dtype=np.float32))
    Wq = fp8.e4m3_encode(np.array([[1, 0, 0, 0], [0, 1, 0, 0], [1, 1, 1, 1]], dtype=np.float32))
    hs = np.array([1.0, 2.0], np.float32)
    ws = np.array([1.0, 0.5, 1.0], np.float32)
    lp, lse = fp8.lmhead_logprob_fp8(Hq, hs, Wq, ws, np.array([2, 0]))
    z0 = np.array([1.0, 1.0, 2.0])            # token 0: (1, 2*0.5, 1+2+0-1)
    z1 = np.array([0.0, 0.0, 8.0])            # token 1: 2*(0, 0, 4)
    want0 = z0[2] - math.log(np.exp(z0).sum())
    want1 = z1[0] - math.log(np.exp(z1).sum())
    assert abs(lp[0] - want0) <= 1e-14 and abs(lp[1] - want1) <= 1e-14


def test_fp8_logprob_is_the_head_on_dequantised_rows():
    rng = np.random.default_rng(1)
    H = rng.standard_normal((40, 128)).astype(np.float32)
    W = (rng.standard_normal((300, 128)) * 0.05).astype(np.float32)
    y = rng.integers(0, 300, 40)
    Hq, hs = fp8.quantize_rows_fp8(H)
    Wq, ws = fp8.quantize_rows_fp8(W)
    lp, lse = fp8.lmhead_logprob_fp8(Hq, hs, Wq, ws, y)
    Hd = np.array([[_value_by_definition(int(c)) for c in row] for row in Hq]) * hs[:, None]
    Wd = np.array([[_value_by_definition(int(c)) for c in row] for row in Wq]) * ws[:, None]
    lp2, lse2 = oracle.lmhead_logprob(Hd, Wd, y)
    assert np.allclose(lp, lp2, rtol=0, atol=1e-12) and np.allclose(lse, lse2, rtol=0, atol=1e-12)
    # and near the unquantised head (3 mantissa bits: a few hundredths here)
    lp3, _ = oracle.lmhead_logprob(H, W, y)
    assert np.max(np.abs(lp - lp3)) < 0.2
