"""The range of the int16 path's digit split, and the input bound that keeps
rotated values inside it (both stated in include/prefill_attn.h).

The int16 scores are formed from int8 digit products (the MNN-on-K3 blog,
§三: an operand wider than the matrix unit's type is split into 8-bit digits
and the partial products recombined exactly): a = 128 h + l with l in
[-64, 63], the digits h and l each stored as int8, and the score recombined
from the products hh, ll and hl + lh.  These tests fix, from that definition
alone, the exact set of a for which both digits fit, and check the documented
sufficient input bound |x| <= 11500 against the Q1.14 tables the oracle
builds.  The GPU tests (test_gpu_range.py) then pin the kernel at the edges:
16319 and -16448 exact, 16320 and -16449 flagged.
"""

import numpy as np

import oracle

LO, HI = -16448, 16319


def _digits(a):
    a = np.asarray(a, dtype=np.int64)
    l = ((a + 64) & 127) - 64
    h = (a - l) >> 7
    return h, l


def _fits(a):
    h, l = _digits(a)
    return (h >= -128) & (h <= 127) & (l >= -64) & (l <= 63)


def test_digits_reconstruct_every_value():
    a = np.arange(-50000, 50001)
    h, l = _digits(a)
    assert np.array_equal(128 * h + l, a)
    assert l.min() == -64 and l.max() == 63


def test_digit_products_recombine_the_score():
    """2^14 hh + 2^7 (hl + lh) + ll is the product of the two values, for
    every pair of the range's edges and a random sample."""
    rng = np.random.default_rng(0)
    a = np.concatenate([[LO, LO + 1, -1, 0, 1, HI - 1, HI], rng.integers(LO, HI + 1, 20000)])
    b = np.concatenate([[HI, LO, 0, -1, 1, LO, HI], rng.integers(LO, HI + 1, 20000)])
    ha, la = _digits(a)
    hb, lb = _digits(b)
    assert np.array_equal((ha * hb << 14) + ((ha * lb + la * hb) << 7) + la * lb, a * b)


def test_contiguous_range_of_exact_digits():
    a = np.arange(LO, HI + 1)
    assert _fits(a).all()
    # the first values outside wrap the h digit
    assert not _fits(HI + 1) and not _fits(LO - 1)
    assert _digits(HI + 1) == (128, -64)
    assert _digits(LO - 1) == (-129, 63)


def test_input_bound_keeps_rotated_values_in_range():
    """With |x|, |y| <= 11500 the fixed-point rotation (x C - y S + 2^13) >> 14
    stays in [LO, HI]: its magnitude is at most (11500 (|C| + |S|) + 2^13) >> 14,
    and |C| + |S| <= 16384 (|cos| + |sin|) + 1 <= 16384 sqrt 2 + 1 for any
    angle (each entry rounded to the nearest integer).  Checked on a dense
    sweep of angles and on the oracle's own tables."""
    bound = int(16384 * np.sqrt(2.0) + 1.0)
    assert ((11500 * bound + 8192) >> 14) <= HI and ((-11500 * bound + 8192) >> 14) >= LO
    ang = np.linspace(0.0, 2.0 * np.pi, 2_000_001)
    rc = np.abs(np.floor(16384.0 * np.cos(ang) + 0.5)) + np.abs(np.floor(16384.0 * np.sin(ang) + 0.5))
    assert rc.max() <= bound
    for D, theta in ((64, 1e4), (128, 1e6)):
        C, S = oracle.rope_table_q14(2048, D, theta)
        assert (np.abs(C) + np.abs(S)).max() <= bound
    # and the bound is close to tight: at 45 degrees 11540 leaves the range
    assert ((11540 * 2 * 11585 + 8192) >> 14) > HI
