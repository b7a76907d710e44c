"""Per-token int16 quantisation of float Q/K feeding the int16 path: plain definition.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Pages (title and section):

* the 2kiu.com/news/6082051 retelling, §3.3: activations (the Q/K/V vectors)
  get a dynamic scale per token, scale_i = 2047 / max(|min_i|, |max_i|), so a
  token with a long tail does not lose the precision of the others; values
  live in the signed 12-bit range [-2048, 2047]; the RoPE table and the
  model-conversion script (§4.2) round with ``np.round`` and clip to that range.
* the MNN-on-K3 blog, §四: the absmax scan, the scale and the quantise-and-pack
  step are done in one pass over the input.

Definitions used here:

1. A row is the D-element vector of one (batch, token, head).  Its absmax
   m = max |x| is exact in fp32.  The scale is fp32(2047 / m) (IEEE division),
   each code is round-half-to-even(fp32(x * scale)) clipped to [-2048, 2047].
   A row of zeros gets codes 0 and dequantisation factor 0.  The decision
   that produces an integer is taken in fp32, as the kernel takes it.
2. The dequantisation factor of a row is m / 2047 (x ~ code * m / 2047).
3. Attention: the codes go through the int16 path of :mod:`oracle.fixed_point`
   (integer RoPE with the Q1.14 table, exact int32 scores); the logit of
   (query i, key j) is s_ij * score_scale * (m_q,i / 2047) * (m_k,j / 2047),
   evaluated in fp64, then the causal softmax and P.V of the float oracle.
"""

import math

import numpy as np

from .attention import _check_shapes, _positions, causal_probs
from .fixed_point import rope_rotate_i16, rope_table_q14, scores_i32

QMAX = 2047


def quantize_rows_i16(x):
    """Codes (int64, same shape) and dequantisation factors m / 2047 (fp64,
    shape x.shape[:-1]) of every last-axis row of x (float values exact in fp32)."""
    x32 = np.asarray(x, dtype=np.float32)
    m = np.max(np.abs(x32), axis=-1)
    codes = np.zeros(x32.shape, dtype=np.int64)
    nz = m > 0
    with np.errstate(divide="ignore"):
        scale = np.where(nz, np.float32(QMAX) / np.where(nz, m, np.float32(1)), np.float32(0)).astype(np.float32)
    prod = (x32 * scale[..., None]).astype(np.float32)
    codes = np.clip(np.rint(prod), -QMAX - 1, QMAX).astype(np.int64)
    codes[~nz] = 0
    inv = m.astype(np.float64) / QMAX
    return codes, inv


def attention_i16_quantized(q, k, v, pos_offsets=None, rope_theta=10000.0, score_scale=None):
    """Float Q/K quantised per (token, head) row, then the int16 path.

    q: [B][S][Hq][D], k: [B][S][Hkv][D] (float values exact in fp32), v float.
    score_scale defaults to 1/sqrt(D).  Returns O float64 [B][S][Hq][D].
    """
    v = np.asarray(v, dtype=np.float64)
    B, S, Hq, Hkv, D = _check_shapes(np.asarray(q), np.asarray(k), v)
    if score_scale is None:
        score_scale = 1.0 / math.sqrt(D)
    g = Hq // Hkv
    qc, qi = quantize_rows_i16(q)
    kc, ki = quantize_rows_i16(k)
    pos = _positions(pos_offsets, B, S)
    table = rope_table_q14(int(pos.max()) + 1, D, rope_theta)
    out = np.zeros((B, S, Hq, D), dtype=np.float64)
    for b in range(B):
        qr = rope_rotate_i16(qc[b], pos[b], rope_theta, table)
        kr = rope_rotate_i16(kc[b], pos[b], rope_theta, table)
        for h in range(Hq):
            kv = h // g
            s = scores_i32(qr[:, h, :], kr[:, kv, :]).astype(np.float64)
            logits = s * float(score_scale) * qi[b, :, h][:, None] * ki[b, :, kv][None, :]
            out[b, :, h, :] = causal_probs(logits) @ v[b, :, kv, :]
    return out


def attention_i16_quantized_rows(q, k, v, rows, pos_offsets=None, rope_theta=10000.0, score_scale=None):
    """:func:`attention_i16_quantized` for selected output rows (b, h, i)."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, S, Hq, Hkv, D = _check_shapes(q, k, v)
    if score_scale is None:
        score_scale = 1.0 / math.sqrt(D)
    g = Hq // Hkv
    pos = _positions(pos_offsets, B, S)
    table = rope_table_q14(int(pos.max()) + 1, D, rope_theta)
    rows = list(rows)
    out = np.zeros((len(rows), D), dtype=np.float64)
    for n, (b, h, i) in enumerate(rows):
        kv = h // g
        qc, qi = quantize_rows_i16(q[b, i:i + 1, h:h + 1, :])
        kc, ki = quantize_rows_i16(k[b, : i + 1, kv:kv + 1, :])
        qr = rope_rotate_i16(qc, pos[b, i:i + 1], rope_theta, table)[0, 0]
        kr = rope_rotate_i16(kc, pos[b, : i + 1], rope_theta, table)[:, 0]
        s = scores_i32(qr[None, :], kr)[0].astype(np.float64)
        lg = s * float(score_scale) * qi[0, 0] * ki[:, 0]
        e = np.exp(lg - lg.max())
        out[n] = (e @ np.asarray(v[b, : i + 1, kv, :], dtype=np.float64)) / e.sum()
    return out
