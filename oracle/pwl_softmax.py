"""Fixed-point-style softmax of the int16 path: piecewise-linear exp and a
Newton reciprocal.  Plain fp64 definition.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Page: the 2kiu.com/news/6082051 retelling, §3.3: exp has no fixed-point
instruction, so x in [-8, 8] is cut into 16 segments and each segment uses a
straight line y = a x + b; the normalising division is not available either.
The page does not print the coefficients.  Definitions used here:

1. Segments: the 16 unit intervals [k, k+1), k = -8 .. 7.  The line of a
   segment is the chord through the knots (k, e^k) and (k+1, e^(k+1)):
   E(t) = e^k * (1 + (e - 1) * (t - k)) for k = floor(t).  E(t) = 0 for
   t < -8; t >= 8 does not occur after the max is subtracted.  (The chord is
   the only line the page's constraints fix without a fitting criterion; it
   is exact at every knot.)
2. Softmax of one query row: x_j = s_j * score_scale for the visible keys,
   m = max_j x_j, w_j = E(x_j - m) (so the largest weight is exactly 1), and
   1 / sum_j w_j by Newton-Raphson division: write l = f * 2^e with f in
   [0.5, 1), start from r0 = 48/17 - 32/17 * f (the classic linear seed,
   error at most 1/17), iterate r <- r * (2 - f * r) three times, then scale
   by 2^-e.
3. O_i = (sum_j w_j V_j) * r.
"""

import math

import numpy as np

from .attention import _check_shapes, _positions
from .fixed_point import rope_rotate_i16, rope_table_q14, scores_i32

SEGMENT_LO = -8
SEGMENTS = 16
NEWTON_STEPS = 3


def pwl_exp(t):
    """E(t): chords of e^x at integer knots on [-8, 8); 0 below -8 (fp64)."""
    t = np.asarray(t, dtype=np.float64)
    out = np.zeros(t.shape, dtype=np.float64)
    ok = t >= SEGMENT_LO
    k = np.floor(t[ok])
    k = np.minimum(k, SEGMENT_LO + SEGMENTS - 1)
    out[ok] = np.exp(k) * (1.0 + (math.e - 1.0) * (t[ok] - k))
    return out


def newton_reciprocal(l):
    """1/l by three Newton-Raphson steps from the 48/17 - 32/17 f seed (l > 0)."""
    l = np.asarray(l, dtype=np.float64)
    f, e = np.frexp(l)  # l = f * 2^e, f in [0.5, 1)
    r = 48.0 / 17.0 - 32.0 / 17.0 * f
    for _ in range(NEWTON_STEPS):
        r = r * (2.0 - f * r)
    return np.ldexp(r, -e)


def pwl_softmax_rows(x, visible):
    """Rows of piecewise-linear softmax weights: x [R][T], visible [R][T] bool.
    Returns (w, r) with w the unnormalised weights and r = 1 / sum w."""
    x = np.where(visible, np.asarray(x, dtype=np.float64), -np.inf)
    m = x.max(axis=1, keepdims=True)
    w = np.where(visible, pwl_exp(np.where(visible, x - m, 0.0)), 0.0)
    return w, newton_reciprocal(w.sum(axis=1))


def attention_i16_pwl(q, k, v, pos_offsets=None, rope_theta=10000.0, score_scale=1.0):
    """int16 Q/K, exact int32 scores, piecewise-linear softmax, P.V in fp64."""
    q = np.asarray(q, dtype=np.int64)
    k = np.asarray(k, dtype=np.int64)
    v = np.asarray(v, dtype=np.float64)
    B, S, Hq, Hkv, D = _check_shapes(q, k, v)
    g = Hq // Hkv
    pos = _positions(pos_offsets, B, S)
    table = rope_table_q14(int(pos.max()) + 1, D, rope_theta)
    causal = np.tril(np.ones((S, S), dtype=bool))
    out = np.zeros((B, S, Hq, D), dtype=np.float64)
    for b in range(B):
        qr = rope_rotate_i16(q[b], pos[b], rope_theta, table)
        kr = rope_rotate_i16(k[b], pos[b], rope_theta, table)
        for h in range(Hq):
            kv = h // g
            x = scores_i32(qr[:, h, :], kr[:, kv, :]).astype(np.float64) * float(score_scale)
            w, r = pwl_softmax_rows(x, causal)
            out[b, :, h, :] = (w @ v[b, :, kv, :]) * r[:, None]
    return out
