"""Pins the piecewise-linear softmax part of the CPU oracle (no GPU).

Knot values and midpoints of the chords, the cut-off below -8, the analytic
worst-case error of a chord of e^x over a unit interval, the accuracy of the
Newton-Raphson reciprocal, integer logits (where the weights are exact), and
the reduction to a plain mean when all scores are equal.
"""

import math

import numpy as np

import oracle
from oracle import pwl_softmax as pw


def test_knots_and_midpoints():
    for k in range(-8, 8):
        assert pw.pwl_exp(np.array([float(k)]))[0] == math.exp(k)
        mid = pw.pwl_exp(np.array([k + 0.5]))[0]
        assert abs(mid - (math.exp(k) + math.exp(k + 1)) / 2) <= 1e-15 * math.exp(k + 1)


def test_cut_off_below_minus_eight():
    assert pw.pwl_exp(np.array([-8.0]))[0] == math.exp(-8)
    assert pw.pwl_exp(np.array([-8.0000001, -9.5, -40.0])).tolist() == [0.0, 0.0, 0.0]


def test_chord_error_bound_is_the_analytic_one():
    # A chord over a unit interval of e^x lies above it; the largest ratio is at
    # f* = (e - 2)/(e - 1): (e - 1) * e^-f* - 1 = 0.1312255...
    f_star = (math.e - 2) / (math.e - 1)
    bound = (math.e - 1) * math.exp(-f_star) - 1
    t = np.linspace(-8, 0, 800001)
    rel = pw.pwl_exp(t) / np.exp(t) - 1
    assert rel.min() >= -1e-15
    assert abs(rel.max() - bound) <= 1e-9
    assert abs(bound - 0.1312255) < 1e-7


def test_newton_reciprocal():
    rng = np.random.default_rng(4)
    l = np.concatenate([[1.0, 2.0, 3.0, 1024.0, 0.75], 10 ** rng.uniform(-3, 6, 2000)])
    r = pw.newton_reciprocal(l)
    assert np.all(np.abs(r * l - 1) <= 1e-9)


def test_integer_logits_give_exact_weights():
    x = np.array([[0.0, -1.0, -3.0, -6.0, 2.0]])  # within 8 of the max
    w, r = pw.pwl_softmax_rows(x, np.ones_like(x, dtype=bool))
    want = np.exp(x - 2.0)
    np.testing.assert_allclose(w, want, rtol=1e-15, atol=0)
    np.testing.assert_allclose(w * r[:, None], want / want.sum(), rtol=1e-9, atol=0)


def test_equal_scores_average_the_values():
    rng = np.random.default_rng(8)
    B, S, Hq, Hkv, D = 1, 12, 2, 1, 16
    q = np.zeros((B, S, Hq, D), dtype=np.int64)  # every score is 0
    k = rng.integers(-2048, 2048, (B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    o = oracle.attention_i16_pwl(q, k, v, score_scale=1e-3)
    for i in range(S):
        np.testing.assert_allclose(o[0, i, 0], v[0, : i + 1, 0].mean(axis=0), rtol=0, atol=1e-9)


def test_tracks_exact_softmax_within_the_chord_bound():
    rng = np.random.default_rng(9)
    B, S, Hq, Hkv, D = 1, 40, 2, 2, 32
    q = rng.integers(-2048, 2048, (B, S, Hq, D))
    k = rng.integers(-2048, 2048, (B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    scale = 2.0 ** -22 / math.sqrt(D) * 8
    a = oracle.attention_i16_pwl(q, k, v, score_scale=scale)
    b = oracle.attention_i16(q, k, v, score_scale=scale)
    # Weights are within a factor 1.132 of exp: O moves by at most ~0.27 max|V|.
    d = np.abs(a - b)
    assert 0 < d.max() <= 0.27 * np.abs(v).max()
