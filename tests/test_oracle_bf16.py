"""Pins of the oracle's bf16 decoding and rounding (oracle/bf16.py) against fixed bit patterns of
the format, and the acceptance and rotary-embedding results that depend on them.

The format: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits, the upper half of an IEEE
binary32.  Rounding is to nearest with ties to the even pattern.  Every expected pattern below is
worked out by hand from those fields, so a truncating rounder, a shift by the wrong amount, a
wrong bias or a tie broken away from even fails one of them.
"""

import numpy as np

import oracle
from oracle import bf16


def test_decode_fixed_patterns():
    cases = {
        0x3F80: 1.0,                       # exponent 127, fraction 0
        0xC000: -2.0,                      # sign, exponent 128
        0x3FC0: 1.5,                       # fraction 0b1000000
        0x3E80: 0.25,
        0x4049: 3.140625,                  # 2 * (1 + 73/128)
        0x0001: 2.0 ** -133,               # smallest subnormal
        0x0080: 2.0 ** -126,               # smallest normal
        0x007F: 127 * 2.0 ** -133,         # largest subnormal
        0x7F7F: (2 - 2 ** -7) * 2.0 ** 127,  # largest finite
        0x8000: -0.0,
        0x0000: 0.0,
    }
    got = bf16.decode(np.array(list(cases), np.uint16))
    assert got.tolist() == list(cases.values())
    assert np.signbit(bf16.decode(np.array([0x8000], np.uint16)))[0]
    inf = bf16.decode(np.array([0xFF80, 0x7F80, 0x7FC0], np.uint16))
    assert inf[0] == -np.inf and inf[1] == np.inf and np.isnan(inf[2])


def test_round_fixed_patterns():
    e8 = 2.0 ** -8
    cases = [
        (1.0, 0x3F80),
        (1 + e8, 0x3F80),                  # halfway between 0x3F80 and 0x3F81: to even (down)
        (1 + 3 * e8, 0x3F82),              # halfway between 0x3F81 and 0x3F82: to even (up)
        (1 + e8 + 2.0 ** -20, 0x3F81),     # just above halfway: up (truncation gives 0x3F80)
        (1 + e8 - 2.0 ** -20, 0x3F80),     # just below halfway: down
        (1 + 2.0 ** -7 - 2.0 ** -30, 0x3F81),   # nearest is above (truncation gives 0x3F80)
        (2 - 2.0 ** -9, 0x4000),           # rounds up across the binade: carry into the exponent
        (2 - 2.0 ** -7, 0x3FFF),           # exactly representable: 1 + 127/128
        (3.14159265358979, 0x4049),        # pi -> 3.140625 (the next pattern 3.15625 is farther)
        (0.1, 0x3DCD),                     # 0.1 = 1.6 * 2^-4: fraction round(0.6 * 128) = 77
        (2.0 ** -133, 0x0001),
        (1.5 * 2.0 ** -133, 0x0002),       # subnormal tie: to even (up)
        (2.5 * 2.0 ** -133, 0x0002),       # subnormal tie: to even (down)
        (2.0 ** -126 - 2.0 ** -134, 0x0080),    # rounds up into the smallest normal
        (0.4 * 2.0 ** -133, 0x0000),
        ((2 - 2 ** -7) * 2.0 ** 127, 0x7F7F),
        ((2 - 2 ** -8) * 2.0 ** 127, 0x7F80),   # halfway above the largest finite: infinity
        (np.inf, 0x7F80),
        (0.0, 0x0000),
    ]
    xs = np.array([c[0] for c in cases])
    want = [c[1] for c in cases]
    assert bf16.round_rne(xs).tolist() == want
    # negatives mirror the positives with the sign bit set
    assert bf16.round_rne(-xs).tolist() == [w | 0x8000 for w in want]
    assert bf16.round_rne(np.array([np.nan])).tolist() == [0x7FC0]


def test_round_is_nearest_on_random_values():
    # against brute force over the neighbouring patterns (decoded exactly): the result is the
    # nearest finite pattern of the same sign, and on an exact tie the one with the even last bit
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(2000) * 2.0 ** -128])
    bits = bf16.round_rne(x).astype(np.int64)
    mag, sign = bits & 0x7FFF, bits & 0x8000
    v = bf16.decode(bits.astype(np.uint16))
    dv = np.abs(x - v)
    up = bf16.decode((sign | np.minimum(mag + 1, 0x7F80)).astype(np.uint16))
    down = bf16.decode((sign | np.maximum(mag - 1, 0)).astype(np.uint16))
    for w in (up, down):
        dw = np.abs(x - w)
        assert np.all(dv <= dw)
        tie = (dv == dw) & (w != v)
        assert np.all(bits[tie] % 2 == 0)


def test_round_matches_the_input_generator_on_fp32_values():
    # the input generator rounds fp32 draws with its own bit trick; on fp32 values (exact in fp64)
    # both roundings must agree
    from synth.gen import f32_to_bf16_bits
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(100000) * 3).astype(np.float32)
    x[:4] = [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 - 2 ** -9]
    assert np.array_equal(bf16.round_rne(x.astype(np.float64)), f32_to_bf16_bits(x))


def test_decode_round_trip():
    pats = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    vals = bf16.decode(pats)
    finite = np.isfinite(vals)
    back = bf16.round_rne(vals[finite])
    # every finite pattern round-trips, -0 included
    assert np.array_equal(back, pats[finite])


def _static_chain():
    # root with two children (tokens 1, 2), each a leaf
    return oracle.build_static([[0], [1]], 2, 1)


def test_accept_uniform_row_bf16_same_as_fp32():
    # a uniform row: p = 1/V > delta/V = min(eps, delta e^-H) (H = ln V), so both children pass,
    # in bf16 exactly as in fp32 (1.5 is exact in both)
    st = _static_chain()
    V = 64
    for dtype in ("f32", "bf16"):
        row = np.full((1, 3, V), 1.5, np.float32)
        logits = bf16.round_rne(row.astype(np.float64)) if dtype == "bf16" else row
        res = oracle.typical_accept(logits, dtype, [[0, 1, 2]], st, 0.7)
        assert res["accepted"][0].tolist() == [True, True, True]
        assert abs(res["entropy"][0, 0] - np.log(V)) < 1e-12
        assert abs(res["threshold"][0, 0] - 0.3 / V) < 1e-15


def test_accept_two_point_row_bf16_same_as_fp32():
    # two equal logits and -inf elsewhere: p = 1/2, H = ln 2, thr = min(0.09, 0.15) = 0.09, so
    # both children pass; in bf16 the -inf is pattern 0xFF80 and 2.0 is 0x4000
    st = _static_chain()
    V = 16
    row32 = np.full((1, 3, V), -np.inf, np.float32)
    row32[0, 0, [1, 2]] = 2.0
    row16 = np.full((1, 3, V), 0xFF80, np.uint16)
    row16[0, 0, [1, 2]] = 0x4000
    for dtype, logits in (("f32", row32), ("bf16", row16)):
        res = oracle.typical_accept(logits, dtype, [[0, 1, 2]], st, 0.7)
        assert res["accepted"][0].tolist() == [True, True, True]
        assert abs(res["entropy"][0, 0] - np.log(2)) < 1e-12
        assert res["threshold"][0, 0] == 0.09
        assert res["accept_length"][0] == 1 and res["best_candidate"][0] == 0


def test_accept_bf16_decisions_use_the_decoded_values():
    # a bf16 row whose decoded values make child 1 pass and child 2 fail; read as if the patterns
    # were shifted by 8 instead of 16 (a plausible slip) the row would be nearly flat and both
    # would pass
    st = _static_chain()
    V = 8
    vals = np.array([0.0, 4.0, -4.0, 0.0, 0.0, 0.0, 0.0, 0.0])
    row = np.zeros((1, 3, V), np.uint16)
    row[0, 0] = bf16.round_rne(vals)
    assert row[0, 0, :3].tolist() == [0x0000, 0x4080, 0xC080]
    res = oracle.typical_accept(row, "bf16", [[0, 1, 2]], st, 1.0)
    p = np.exp(vals) / np.exp(vals).sum()
    H = -(p * np.log(p)).sum()
    thr = min(0.09, 0.3 * np.exp(-H))
    assert p[1] > thr and p[2] < thr
    assert res["accepted"][0].tolist() == [True, True, False]
