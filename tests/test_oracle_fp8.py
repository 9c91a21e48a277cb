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


# --- MXFP4 ---

def test_e2m1_table_and_round_trip():
    # the 16 codes by their bit fields: sign, 2 exponent bits (bias 1), 1 mantissa bit
    for c in range(16):
        s = -1.0 if c & 8 else 1.0
        e, m = (c >> 1) & 3, c & 1
        want = s * (m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1))
        assert fp8.e2m1_decode(c) == want, c
    codes = np.arange(16, dtype=np.uint8)
    back = fp8.e2m1_encode(fp8.e2m1_decode(codes).astype(np.float32))
    assert np.array_equal(back[codes != 8], codes[codes != 8]) and back[8] == 8  # -0 keeps its sign


@pytest.mark.parametrize("x,code", [
    (0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),   # ties to even
    (0.3, 1), (2.9, 5), (4.9, 6), (5.1, 7), (7.0, 7), (100.0, 7), (-1.0, 10), (-0.0, 8),
])
def test_e2m1_roundings(x, code):
    assert int(fp8.e2m1_encode(np.float32(x))) == code


def test_mxfp4_block_scales_by_hand():
    # block 0: amax 6 -> 2^(2 - 2) = 1 (code 127), values exact; block 1: amax 0.75 -> 2^(-1 - 2)
    # = 1/8 (code 124), 0.75 * 8 = 6 exact; block 2 all zero -> code 0; block 3: amax 1000 ->
    # 2^(9 - 2) = 128 (code 134), 1000 / 128 = 7.8 saturates to 6
    X = np.zeros((1, 128), np.float32)
    X[0, :8] = [6, -4, 3, 1.5, 1, 0.5, 0, -6]
    X[0, 32] = 0.75
    X[0, 33] = -0.0625  # 0.5 after scaling
    X[0, 96] = 1000.0
    X[0, 97] = 64.0     # 0.5 after scaling
    q, s = fp8.quantize_rows_mxfp4(X)
    assert list(s[0]) == [127, 124, 0, 134]
    back = fp8.mxfp4_decode(q, s)[0]
    assert list(back[:8]) == [6, -4, 3, 1.5, 1, 0.5, 0, -6]
    assert back[32] == 0.75 and back[33] == -0.0625
    assert back[96] == 768.0 and back[97] == 64.0
    assert np.all(back[64:96] == 0)
    # packing: element 0 in the low nibble of byte 0
    assert q[0, 0] & 15 == 7 and q[0, 0] >> 4 == 14  # 6 -> 7, -4 -> 8|6


def test_mxfp4_error_bound():
    """Every element is within half an E2M1 step of its block's scaled grid:
    |x - q| <= 2^e * (step at |x| / 2^e) / 2, at most 2^e for the top binade,
    and saturated values are within 2 * 2^e of 6 * 2^e."""
    rng = np.random.default_rng(2)
    X = rng.standard_normal((20, 256)).astype(np.float32)
    q, s = fp8.quantize_rows_mxfp4(X)
    back = fp8.mxfp4_decode(q, s).reshape(20, 8, 32)
    sc = np.ldexp(1.0, s.astype(np.int64) - 127)[:, :, None]
    err = np.abs(back - X.reshape(20, 8, 32)) / sc
    assert np.all(err <= 2.0 + 1e-12)
    assert np.all(np.max(np.abs(back), axis=2) / sc[:, :, 0] >= 4.0)  # the block maximum uses the top binade


def test_mxfp4_logprob_is_the_head_on_decoded_rows():
    rng = np.random.default_rng(3)
    H = rng.standard_normal((30, 128)).astype(np.float32)
    W = (rng.standard_normal((200, 128)) * 0.05).astype(np.float32)
    y = rng.integers(0, 200, 30)
    Hq, hs = fp8.quantize_rows_fp8(H)
    Wq, ws = fp8.quantize_rows_mxfp4(W)
    lp, lse = fp8.lmhead_logprob_mxfp4(Hq, hs, Wq, ws, y)
    Hd = np.array([[_value_by_definition(int(c)) for c in row] for row in Hq]) * hs[:, None]
    Wd = np.zeros((200, 128))
    for r in range(200):
        for k in range(128):
            nib = (Wq[r, k // 2] >> (4 * (k % 2))) & 15
            Wd[r, k] = fp8.e2m1_decode(nib) * 2.0 ** (int(ws[r, k // 32]) - 127)
    lp2, lse2 = oracle.lmhead_logprob(Hd, Wd, y)
    assert np.allclose(lp, lp2, rtol=0, atol=1e-12) and np.allclose(lse, lse2, rtol=0, atol=1e-12)
