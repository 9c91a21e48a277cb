"""Oracle: FP8 (E4M3) head -- per-row quantisation and the sampled-token
logprob from FP8 operands (float64, CPU).

TEST INFRASTRUCTURE -- see the package docstring for who may use it.

Source: "vLLM says aligned kernels make asynchronous RL stable at lag 64",
section "Zero mismatch expands to newer models": the consistent path of the
newest model uses FP8 (and MXFP4) weights, so the aligned logprob must hold
for a low-precision head too. The pages give no format details; readings:

* Format: OCP 8-bit E4M3 ("E4M3FN"): 1 sign bit, 4 exponent bits (bias 7),
  3 mantissa bits, subnormals, no infinities, largest finite value 448.
* Per-row scaling (a row of W is one vocabulary entry, a row of H one
  token): scale = amax / 448 in float32 (1 for an all-zero row), code =
  E4M3 of x / scale, the division in float32 and the conversion rounding to
  nearest, ties to even, saturating at +-448. Every step is IEEE float32 (or
  exact), so the codes are a fixed function of the input bits.
* Logits: z[t, v] = h_scale[t] * w_scale[v] * sum_k e4m3(Hq[t, k]) *
  e4m3(Wq[v, k]); then the same log-softmax and gather as the bf16 head.

Pins (tests/test_oracle_fp8.py): every one of the 254 finite codes
round-trips through decode and encode; hand-picked values (1 -> 0x38,
448 -> 0x7E, 2^-9 -> 0x01, ties at the subnormal and normal scale go to the
even code, 460 -> 448, 480 and beyond saturate); scales of hand-made rows;
an all-zero row; the fp8 logprob against the bf16 oracle on the decoded,
rescaled operands and on a tiny head where every value is exact.
"""

import numpy as np

from .lmhead import lmhead_logprob

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Exact float64 values of E4M3 codes (uint8). 0x7F / 0xFF (NaN) decode
    to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    v = np.where(e == 0, np.ldexp(m, -9), np.ldexp(1.0 + m / 8.0, e - 7))
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return s * v


def e4m3_encode(x):
    """E4M3 codes of float32 values: round to nearest, ties to even,
    saturating at +-448 (NaN is not expected and encodes as 0x7F)."""
    x = np.asarray(x, dtype=np.float32)
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.abs(x).astype(np.float64)  # exact
    out = np.zeros(x.shape, dtype=np.uint8)
    # subnormal range: multiples of 2^-9 below 2^-6
    sub = a < 2.0 ** -6
    ms = np.rint(np.ldexp(a[sub], 9))  # ties to even; 8 becomes the smallest normal, code 0x08
    out[sub] = ms.astype(np.uint8)
    nor = ~sub
    an = a[nor]
    e = np.floor(np.log2(an)).astype(np.int64)
    # guard log2 rounding: make 2^e <= a < 2^(e+1) exact
    e = np.where(np.ldexp(1.0, e) > an, e - 1, e)
    e = np.where(np.ldexp(1.0, e + 1) <= an, e + 1, e)
    r = np.rint(np.ldexp(an, 3 - e))  # in [8, 16], ties to even
    carry = r == 16
    e = np.where(carry, e + 1, e)
    r = np.where(carry, 8, r)
    code = ((e + 7) << 3) | (r.astype(np.int64) - 8)
    code = np.where((e > 8) | ((e == 8) & (r > 14)), 0x7E, code)  # saturate at 448 = 2^8 * 1.75
    out[nor] = code.astype(np.uint8)
    out |= sign
    out = np.where(np.isnan(x), np.uint8(0x7F), out)
    return out


def quantize_rows_fp8(X):
    """Per-row E4M3 quantisation of a float32-representable matrix (bf16
    bit patterns as uint16 or float arrays): returns (codes uint8 [n, d],
    scale float32 [n])."""
    from .lmhead import to_f64

    Xf = to_f64(X).astype(np.float32)  # bf16 and fp32 values are exact in float32
    amax = np.max(np.abs(Xf), axis=1) if Xf.shape[1] else np.zeros(Xf.shape[0], np.float32)
    scale = np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32), np.float32(1.0)).astype(np.float32)
    q = e4m3_encode((Xf / scale[:, None]).astype(np.float32))
    return q, scale


def lmhead_logprob_fp8(Hq, h_scale, Wq, w_scale, tokens, vocab_chunk=8192):
    """Sampled-token logprob and lse from E4M3 operands with per-row
    scales: the bf16 head's definition applied to the exact decoded values,
    each row multiplied by its scale."""
    Hd = e4m3_decode(Hq) * np.asarray(h_scale, dtype=np.float64)[:, None]
    Wd = e4m3_decode(Wq) * np.asarray(w_scale, dtype=np.float64)[:, None]
    return lmhead_logprob(Hd, Wd, tokens, vocab_chunk=vocab_chunk)


# --- MXFP4 weights (OCP Microscaling: FP4 E2M1 elements, E8M0 block scales) ---
#
# Same section of the same page ("FP8 and MXFP4 weights"). Readings: the OCP
# MX format, blocks of 32 consecutive values along the contraction dimension
# (d) sharing one power-of-two scale 2^e stored as E8M0 (e + 127); the scale
# of a block is 2^(floor(log2 amax) - 2) (2 = the exponent of E2M1's largest
# value, 6 = 1.5 x 2^2), clamped to [2^-127, 2^127], and 2^-127 (code 0) for
# an all-zero block; elements are E2M1 of x / 2^e (exact power-of-two
# scaling), rounding to nearest, ties to even, saturating at +-6. Codes are
# packed two per byte, element k in the low nibble when k is even. Against an
# MXFP4 head the activations are E4M3 with per-row scales, as above.

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes):
    """Exact values of E2M1 codes (low 4 bits of each entry)."""
    c = np.asarray(codes).astype(np.int64) & 15
    v = E2M1_VALUES[c & 7]
    return np.where(c & 8, -v, v)


def e2m1_encode(x):
    """E2M1 codes of float32 values: round to nearest, ties to even,
    saturating at +-6."""
    x = np.asarray(x, dtype=np.float32)
    sign = (np.signbit(x)).astype(np.uint8) << 3
    a = np.abs(x).astype(np.float64)
    out = np.zeros(x.shape, dtype=np.uint8)
    sub = a < 1.0
    out[sub] = np.rint(a[sub] * 2.0).astype(np.uint8)  # 0, 0.5 or (rounded up) 1.0 = code 2
    nor = ~sub
    an = a[nor]
    e = np.floor(np.log2(an)).astype(np.int64)
    e = np.where(np.ldexp(1.0, e) > an, e - 1, e)
    e = np.where(np.ldexp(1.0, e + 1) <= an, e + 1, e)
    r = np.rint(np.ldexp(an, 1 - e))  # in [2, 4], ties to even
    carry = r == 4
    e = np.where(carry, e + 1, e)
    r = np.where(carry, 2, r)
    code = ((e + 1) << 1) | (r.astype(np.int64) - 2)
    code = np.where((e > 2) | ((e == 2) & (r > 3)), 7, code)
    out[nor] = code.astype(np.uint8)
    return out | sign


def quantize_rows_mxfp4(X):
    """MXFP4 of a matrix [n, d] (d a multiple of 32): (packed codes uint8
    [n, d/2], E8M0 scale codes uint8 [n, d/32])."""
    from .lmhead import to_f64

    Xf = to_f64(X).astype(np.float32)
    n, d = Xf.shape
    blocks = Xf.reshape(n, d // 32, 32)
    amax = np.max(np.abs(blocks), axis=2).astype(np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    e = np.floor(np.log2(safe)).astype(np.int64)
    e = np.where(np.ldexp(1.0, e) > safe, e - 1, e)
    e = np.where(np.ldexp(1.0, e + 1) <= safe, e + 1, e)
    e = np.clip(e - 2, -127, 127)
    e = np.where(amax > 0, e, -127)
    scaled = np.ldexp(blocks.astype(np.float64), -e[:, :, None]).astype(np.float32)  # exact
    codes = e2m1_encode(scaled).reshape(n, d)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def mxfp4_decode(packed, scale_codes):
    """Exact float64 values of an MXFP4 matrix."""
    p = np.asarray(packed, dtype=np.uint8)
    n, half = p.shape
    codes = np.empty((n, 2 * half), dtype=np.uint8)
    codes[:, 0::2] = p & 15
    codes[:, 1::2] = p >> 4
    v = e2m1_decode(codes).reshape(n, -1, 32)
    sc = np.ldexp(1.0, np.asarray(scale_codes, dtype=np.int64) - 127)
    return (v * sc[:, :, None]).reshape(n, 2 * half)


def lmhead_logprob_mxfp4(Hq, h_scale, Wq4, w_scale_codes, tokens, vocab_chunk=8192):
    """Sampled-token logprob and lse of an MXFP4 head against E4M3 token
    rows with per-row scales: the head's definition on the exact decoded
    values."""
    Hd = e4m3_decode(Hq) * np.asarray(h_scale, dtype=np.float64)[:, None]
    Wd = mxfp4_decode(Wq4, w_scale_codes)
    return lmhead_logprob(Hd, Wd, tokens, vocab_chunk=vocab_chunk)
