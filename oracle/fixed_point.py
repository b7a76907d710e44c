"""Int16 fixed-point oracle: exact integer RoPE and exact int32 scores.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

The "手写内核实现6倍prefill加速" page (§3.1) does RoPE in the int16 domain:
cos/sin of i*theta_k are looked up in int16 tables of length max seq_len and
the rotation and the q'.k' dot are integer arithmetic.  The 2kiu.com retelling
(§3.3, §4.2) builds the table offline at high precision and rounds it to a
fixed-point format.  The pages disagree on that format (Q12.4 truncation in
the script, "rounding" in §3.3); the variant defined here is:

* tables in Q1.14: C[p][k] = round(cos(p*theta_k) * 2^14),
  S[p][k] = round(sin(p*theta_k) * 2^14), round to nearest with ties away
  from zero (no tie occurs for p >= 1; p = 0 gives C = 16384, S = 0);
* rotation with round-half-up (toward +infinity) and an arithmetic shift:
  x' = (x*C - y*S + 2^13) >> 14,  y' = (x*S + y*C + 2^13) >> 14;
* scores s_ij = sum_d q'_d k'_d, exact in integers (|s| < 2^31 is asserted);
* logits s * score_scale in fp64, then the causal two-pass softmax and P.V of
  the float oracle (V converted exactly to fp64).
"""

import math

import numpy as np

from .attention import _check_shapes, _positions, causal_probs, rope_inv_freq


def _round_nearest_away(x):
    """Round a finite fp64 value to the nearest integer, ties away from zero.

    Exact: the integer part and the fraction are split without rounding.
    """
    n = math.floor(abs(x))
    frac = abs(x) - n          # exact for |x| < 2^52
    r = n + (1 if frac >= 0.5 else 0)
    return r if x >= 0 else -r


def rope_table_q14(n_positions, head_dim, rope_theta):
    """Q1.14 cos/sin tables for positions 0..n_positions-1.

    Returns (C, S), int64 arrays of shape [n_positions][head_dim/2].
    The angle is the fp64 product p * theta_k; cos/sin are the C library's.
    """
    inv = rope_inv_freq(head_dim, rope_theta).tolist()
    half = head_dim // 2
    C = np.empty((n_positions, half), dtype=np.int64)
    S = np.empty((n_positions, half), dtype=np.int64)
    for p in range(n_positions):
        for k in range(half):
            a = float(p) * inv[k]
            C[p, k] = _round_nearest_away(math.cos(a) * 16384.0)
            S[p, k] = _round_nearest_away(math.sin(a) * 16384.0)
    return C, S


def rope_rotate_i16(x, positions, rope_theta, table=None):
    """Integer RoPE of x [S][H][D] (int16 values) at positions [S].

    Returns int64 [S][H][D]; every value is asserted to fit int16.
    ``table`` may pass a precomputed (C, S) covering max(positions)+1 rows.
    """
    x = np.asarray(x, dtype=np.int64)
    Sq, _, D = x.shape
    pos = np.asarray(positions, dtype=np.int64).reshape(-1)
    if table is None:
        table = rope_table_q14(int(pos.max()) + 1 if pos.size else 1, D, rope_theta)
    Ct, St = table
    c = Ct[pos][:, None, :]
    s = St[pos][:, None, :]
    xr = x[..., 0::2]
    xi = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = (xr * c - xi * s + 8192) >> 14
    out[..., 1::2] = (xr * s + xi * c + 8192) >> 14
    if out.size and (out.max() > 32767 or out.min() < -32768):
        raise OverflowError("rotated value does not fit int16")
    return out


def scores_i32(q_rot, k_rot):
    """Exact integer dot products q'_i . k'_j for [S][D] x [S][D] -> [S][S].

    Every product is below 2^24 in magnitude and every partial sum below
    2^53, so the fp64 matrix product is exact; the result is checked to be
    integral and to fit int32.
    """
    qf = np.asarray(q_rot, dtype=np.float64)
    kf = np.asarray(k_rot, dtype=np.float64)
    if qf.size and (np.abs(qf).max() >= 2 ** 15 or np.abs(kf).max() >= 2 ** 15):
        raise ValueError("operands must be int16 values")
    if qf.shape[-1] > 8192:
        raise ValueError("dot length too long for exact fp64 sums")
    s = qf @ kf.T
    si = s.astype(np.int64)
    if not np.array_equal(si.astype(np.float64), s):
        raise ArithmeticError("fp64 score is not integral")
    if si.size and np.abs(si).max() >= 2 ** 31:
        raise OverflowError("score does not fit int32")
    return si


def attention_i16(q, k, v, pos_offsets=None, rope_theta=10000.0, score_scale=1.0):
    """Fixed-point variant: integer RoPE, exact scores, fp64 softmax and P.V.

    q: int16 values [B][S][Hq][D]; k: int16 values [B][S][Hkv][D];
    v: float values [B][S][Hkv][D].  Returns O float64 [B][S][Hq][D].
    """
    q = np.asarray(q, dtype=np.int64)
    k = np.asarray(k, dtype=np.int64)
    v = np.asarray(v, dtype=np.float64)
    B, S, Hq, Hkv, D = _check_shapes(q, k, v)
    g = Hq // Hkv
    pos = _positions(pos_offsets, B, S)
    table = rope_table_q14(int(pos.max()) + 1, D, rope_theta)
    out = np.zeros((B, S, Hq, D), dtype=np.float64)
    for b in range(B):
        qr = rope_rotate_i16(q[b], pos[b], rope_theta, table)
        kr = rope_rotate_i16(k[b], pos[b], rope_theta, table)
        for h in range(Hq):
            kv = h // g
            s = scores_i32(qr[:, h, :], kr[:, kv, :])
            p = causal_probs(s.astype(np.float64) * float(score_scale))
            out[b, :, h, :] = p @ v[b, :, kv, :]
    return out


def attention_i16_rows(q, k, v, rows, pos_offsets=None, rope_theta=10000.0, score_scale=1.0):
    """:func:`attention_i16` for selected output rows (b, h, i) only."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, S, Hq, Hkv, D = _check_shapes(q, k, v)
    g = Hq // Hkv
    pos = _positions(pos_offsets, B, S)
    rows = list(rows)
    table = rope_table_q14(int(pos.max()) + 1, D, rope_theta)
    out = np.zeros((len(rows), D), dtype=np.float64)
    for n, (b, h, i) in enumerate(rows):
        kv = h // g
        qi = rope_rotate_i16(np.asarray(q[b, i:i + 1, h:h + 1, :]), pos[b, i:i + 1], rope_theta, table)[0, 0]
        kk = rope_rotate_i16(np.asarray(k[b, : i + 1, kv:kv + 1, :]), pos[b, : i + 1], rope_theta, table)[:, 0]
        s = scores_i32(qi[None, :], kk)[0]
        lg = s.astype(np.float64) * float(score_scale)
        e = np.exp(lg - lg.max())
        out[n] = (e @ np.asarray(v[b, : i + 1, kv, :], dtype=np.float64)) / e.sum()
    return out
