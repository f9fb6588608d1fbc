"""Oracle: bfloat16 storage format, decoding and rounding (fp64, numpy).  Test infrastructure only.

The bf16 workloads hold every tensor as bfloat16 bit patterns (uint16): the upper half of an
IEEE binary32, so 1 sign bit, 8 exponent bits (bias 127) and 7 fraction bits.  The pages fix no
precision beyond "bf16"; the readings used everywhere in the oracle are:
  * decoding is exact: a bf16 value is the binary32 whose upper 16 bits are the pattern and
    whose lower 16 bits are zero;
  * results stored as bf16 (rotated queries and keys, attention outputs on the GPU side) are
    rounded once, from the exact fp64 value, to the nearest bf16, ties to the even pattern;
    magnitudes from the largest finite value plus half an ulp upward become infinity.
This module is the one place in the oracle where bf16 is decoded or rounded.
"""

import numpy as np

SUBNORMAL_ULP = 2.0 ** -133          # spacing of bf16 values below the smallest normal 2^-126


def decode(bits):
    """bf16 bit patterns -> exact fp64 values (same shape)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):          # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def round_rne(x):
    """fp64 values -> bf16 bit patterns (uint16), round to nearest, ties to even, written from
    the format's fields: the sign, then the magnitude as a multiple of the spacing of its binade
    (2^-133 below 2^-126, else 2^(e-8) for a value m * 2^e with 0.5 <= m < 1).  NaN -> 0x7FC0."""
    x = np.asarray(x, np.float64)
    shape = x.shape
    x = x.reshape(-1)
    out = np.zeros(x.shape, np.uint32)
    sign = np.signbit(x).astype(np.uint32) << np.uint32(15)
    a = np.abs(x)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, a)
    sub = a < 2.0 ** -126
    # subnormal range: a multiple q of 2^-133 (q = 128 is the smallest normal, pattern 0x0080)
    q = np.rint(a[sub] / SUBNORMAL_ULP)
    out[sub] = q.astype(np.uint32)
    # normal range: 8 significant bits s in [128, 256) at exponent e - 8
    an = a[~sub]
    big = np.isinf(an)
    m, e = np.frexp(np.where(big, 1.0, an))
    s = np.rint(m * 256.0)
    carry = s == 256.0                 # rounded up into the next binade
    s = np.where(carry, 128.0, s)
    e = e + carry.astype(e.dtype)
    biased = e - 1 + 127               # value = (s / 128) * 2^(e - 1)
    inf = (biased >= 255) | big
    fields = (biased.astype(np.int64) << 7) | (s.astype(np.int64) - 128)
    fields = np.where(inf, 0x7F80, fields)
    out[~sub] = fields.astype(np.uint32)
    out = out | sign
    out[nan] = 0x7FC0
    return out.astype(np.uint16).reshape(shape)


def to_f64(a, dtype):
    """A stored tensor as fp64: bf16 bit patterns (uint16) when dtype is "bf16", else fp32 (or
    already fp64) values."""
    a = np.asarray(a)
    if dtype == "bf16" and a.dtype == np.uint16:
        return decode(a)
    return a.astype(np.float64)
