"""Float oracle: RoPE + causal softmax attention, plain fp64 definition.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What is computed, step by step, in the pages' notation:

1. Position of token i of batch element b: p = off[b] + i.  The pages never
   define position offsets for a prefill; the reading taken is that the
   offset shifts the RoPE position of every query and key token alike and
   the causal mask stays "key j visible to query i iff j <= i".
2. RoPE frequencies theta_k = rope_theta^(-2k/D), k = 0..D/2-1, and the angle
   p*theta_k, in fp64.  (The RoPE table script on the 2kiu.com page, §4.2,
   divides by the model's hidden size; RoPE acts per head, so D here is the
   head dimension.)
3. Each adjacent pair (x, y) = (X[2k], X[2k+1]) is multiplied by the unit
   complex number e^{i p theta_k}: x' = x cos - y sin, y' = x sin + y cos
   ("手写内核实现6倍prefill加速" page, §3.1: RoPE as a complex multiply, real
   part first, imaginary part second).  Q and K are rotated; V is not.
4. Scores Q'_i . K'_j * scale for the query head h and its KV head
   kvh(h) = floor(h / (Hq / Hkv)); keys j > i are masked (causal).
5. Softmax over the visible keys in two passes (row max, then exp and sum),
   then O_i = sum_j P_ij V_j.  The pages fuse this as a blocked online
   softmax with no S x S matrix in memory (2kiu.com page §2.1; MNN-on-K3
   blog §六; XNet-DNN article §三.3); in exact arithmetic that reaches the
   same O, so the oracle forms the full causal score matrix instead.

Tensors are row-major [B][S][H][D]; every array is converted to float64.
"""

import math

import numpy as np


def rope_inv_freq(head_dim, rope_theta):
    """theta_k = rope_theta ** (-2k / head_dim), k < head_dim / 2, in fp64.

    Evaluated with the C library's ``pow`` (``math.pow``) on the fp64
    exponent ``(-2.0 * k) / head_dim``.
    """
    if head_dim % 2:
        raise ValueError("head_dim must be even (RoPE rotates pairs)")
    return np.array(
        [math.pow(float(rope_theta), (-2.0 * k) / head_dim) for k in range(head_dim // 2)],
        dtype=np.float64,
    )


def rope_cos_sin(positions, head_dim, rope_theta):
    """cos and sin of the angle p * theta_k for every position p given.

    Returns two fp64 arrays of shape [len(positions)][head_dim/2].  The angle
    is the fp64 product of the integer position and theta_k; cos and sin are
    the C library's (``math.cos``/``math.sin``).
    """
    inv = rope_inv_freq(head_dim, rope_theta)
    pos = np.asarray(positions, dtype=np.int64).reshape(-1)
    ang = pos.astype(np.float64)[:, None] * inv[None, :]
    flat = ang.reshape(-1).tolist()
    cos = np.array([math.cos(a) for a in flat], dtype=np.float64).reshape(ang.shape)
    sin = np.array([math.sin(a) for a in flat], dtype=np.float64).reshape(ang.shape)
    return cos, sin


def rope_rotate(x, positions, rope_theta):
    """Rotate interleaved pairs of x [S][H][D] by the angles of positions [S]."""
    x = np.asarray(x, dtype=np.float64)
    S, _, D = x.shape
    cos, sin = rope_cos_sin(positions, D, rope_theta)
    c = cos[:, None, :]
    s = sin[:, None, :]
    xr = x[..., 0::2]
    xi = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xr * c - xi * s
    out[..., 1::2] = xr * s + xi * c
    return out


def causal_probs(scores):
    """Causal two-pass softmax of a square score matrix [S][S] (query, key).

    Entries with key j > query i get probability exactly 0.
    """
    sc = np.array(scores, dtype=np.float64, copy=True)
    S = sc.shape[0]
    masked = np.triu(np.ones((S, S), dtype=bool), k=1)
    sc[masked] = -np.inf
    m = sc.max(axis=1, keepdims=True)
    e = np.exp(sc - m)
    e[masked] = 0.0
    l = e.sum(axis=1, keepdims=True)
    return e / l


def _positions(pos_offsets, batch, seq_len):
    if pos_offsets is None:
        off = np.zeros(batch, dtype=np.int64)
    else:
        off = np.asarray(pos_offsets, dtype=np.int64).reshape(-1)
        if off.shape[0] != batch:
            raise ValueError("pos_offsets must have one entry per batch element")
    return off[:, None] + np.arange(seq_len, dtype=np.int64)[None, :]


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B][S][H][D]")
    B, S, Hq, D = q.shape
    if k.shape[:2] != (B, S) or v.shape[:2] != (B, S):
        raise ValueError("q, k, v must share batch and sequence length")
    Hkv = k.shape[2]
    if v.shape[2] != Hkv or k.shape[3] != D or v.shape[3] != D:
        raise ValueError("k and v must be [B][S][Hkv][D] with the q head_dim")
    if Hkv == 0 or Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    return B, S, Hq, Hkv, D


def attention(q, k, v, pos_offsets=None, rope_theta=10000.0, scale=None):
    """O = softmax_causal(RoPE(Q) RoPE(K)^T * scale) V, all in fp64.

    q: [B][S][Hq][D]; k, v: [B][S][Hkv][D]; returns O [B][S][Hq][D] float64.
    scale defaults to 1/sqrt(D).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, S, Hq, Hkv, D = _check_shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    g = Hq // Hkv
    pos = _positions(pos_offsets, B, S)
    out = np.zeros((B, S, Hq, D), dtype=np.float64)
    for b in range(B):
        qr = rope_rotate(q[b], pos[b], rope_theta)
        kr = rope_rotate(k[b], pos[b], rope_theta)
        for h in range(Hq):
            kv = h // g
            sc = (qr[:, h, :] @ kr[:, kv, :].T) * scale
            p = causal_probs(sc)
            out[b, :, h, :] = p @ v[b, :, kv, :]
    return out


def attention_rows(q, k, v, rows, pos_offsets=None, rope_theta=10000.0, scale=None):
    """The same O as :func:`attention`, for selected output rows only.

    rows: iterable of (b, h, i).  Each row needs query i and keys 0..i only,
    so this evaluates the definition one row at a time at any size.
    Returns float64 [len(rows)][D].
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, S, Hq, Hkv, D = _check_shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    g = Hq // Hkv
    pos = _positions(pos_offsets, B, S)
    rows = list(rows)
    out = np.zeros((len(rows), D), dtype=np.float64)
    for n, (b, h, i) in enumerate(rows):
        kv = h // g
        qi = rope_rotate(np.asarray(q[b, i:i + 1, h:h + 1, :], dtype=np.float64), pos[b, i:i + 1], rope_theta)[0, 0]
        kk = rope_rotate(np.asarray(k[b, : i + 1, kv:kv + 1, :], dtype=np.float64), pos[b, : i + 1], rope_theta)[:, 0]
        vv = np.asarray(v[b, : i + 1, kv, :], dtype=np.float64)
        sc = (kk @ qi) * scale
        m = sc.max()
        e = np.exp(sc - m)
        out[n] = (e @ vv) / e.sum()
    return out
