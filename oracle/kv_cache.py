"""KV-prefix (chunked) prefill against a KV cache: plain fp64 definition.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Pages (title and section):

* "手写内核实现6倍prefill加速：边缘LLM推理的内存与计算协同优化", §2.2: the
  cache-update kernel copies only the K/V of the tokens that are new and
  leaves the older entries where they are; §3.2: the ring KV cache stores K/V
  in whatever physical place is free and keeps a small index map with one
  physical offset per logical position, so the attention still reads the keys
  in logical order 0, 1, 2, ...
* the 2kiu.com/news/6082051 retelling, §3.4: a ring of slots whose index wraps
  with a bit mask (slot = index & (n_slots - 1) for a power-of-two ring).

Definitions used here (the pages fix the structure, not these names):

1. A cache is K_cache, V_cache of shape [n_slots][Hkv][D].  For sequence b,
   kv_map[b][j] is the slot that holds logical position j.
2. kv_cache_update: new token i of sequence b has logical position
   P_b + i (P_b = the number of tokens the cache already holds for b) and is
   written to slot kv_map[b][P_b + i]; no other slot changes.
3. Cached prefill: query i of sequence b sits at position P_b + i and attends
   to the logical keys j = 0 .. P_b + i, key j taken from slot kv_map[b][j]
   and rotated at position j.  RoPE, the score scale and the two-pass softmax
   are those of :func:`oracle.attention` (P_b = 0 with the identity map is
   exactly that function's causal prefill).
"""

import math

import numpy as np

from .attention import rope_rotate
from .fixed_point import rope_rotate_i16, rope_table_q14, scores_i32


def ring_index_map(n_slots, start, count):
    """Slots of logical positions 0..count-1 in a ring that starts at `start`:
    (start + j) mod n_slots (for a power of two this is the bit mask of the
    2kiu.com page, §3.4)."""
    return np.array([(start + j) % n_slots for j in range(count)], dtype=np.int64)


def paged_index_map(block_table, block_size, count):
    """Slots of logical positions 0..count-1 when the cache is cut into blocks
    of `block_size` slots and block_table[n] is the physical block that holds
    logical block n: block_table[j // block_size] * block_size + j % block_size."""
    return np.array([block_table[j // block_size] * block_size + j % block_size for j in range(count)],
                    dtype=np.int64)


def _prefix(prefix, batch):
    if prefix is None:
        return np.zeros(batch, dtype=np.int64)
    p = np.asarray(prefix, dtype=np.int64).reshape(-1)
    if p.shape[0] != batch or (p < 0).any():
        raise ValueError("prefix must hold one non-negative length per batch element")
    return p


def kv_cache_update(k_cache, v_cache, k_new, v_new, kv_map, prefix=None):
    """Return copies of the caches with the new tokens written to their slots.

    k_cache, v_cache: [n_slots][Hkv][D]; k_new, v_new: [B][S][Hkv][D];
    kv_map: [B][>= P_b + S] slots; prefix: [B] (None = zeros).
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    k_new = np.asarray(k_new)
    v_new = np.asarray(v_new)
    B, S = k_new.shape[:2]
    p = _prefix(prefix, B)
    kv_map = np.asarray(kv_map, dtype=np.int64)
    written = set()
    for b in range(B):
        for i in range(S):
            slot = int(kv_map[b, p[b] + i])
            if not 0 <= slot < kc.shape[0]:
                raise IndexError("slot out of range")
            if slot in written:
                raise ValueError("two new tokens map to the same slot")
            written.add(slot)
            kc[slot] = k_new[b, i]
            vc[slot] = v_new[b, i]
    return kc, vc


def gather_logical(cache, kv_map, b, count):
    """Logical positions 0..count-1 of sequence b: cache[kv_map[b][j]], [count][Hkv][D]."""
    slots = np.asarray(kv_map, dtype=np.int64)[b, :count]
    return np.asarray(cache)[slots]


def _prefix_probs(scores, shift):
    """Two-pass softmax of scores [S][T] where query i sees keys j <= shift + i."""
    sc = np.array(scores, dtype=np.float64, copy=True)
    S, T = sc.shape
    masked = np.arange(T)[None, :] > (shift + np.arange(S))[:, None]
    sc[masked] = -np.inf
    m = sc.max(axis=1, keepdims=True)
    e = np.exp(sc - m)
    e[masked] = 0.0
    return e / e.sum(axis=1, keepdims=True)


def attention_cached(q, k_cache, v_cache, kv_map, prefix=None, rope_theta=10000.0, scale=None):
    """Cached prefill O [B][S][Hq][D] in fp64 (float inputs).

    q: [B][S][Hq][D] (the new tokens); k_cache, v_cache: [n_slots][Hkv][D]
    already holding every logical position 0 .. P_b + S - 1 of each sequence.
    """
    q = np.asarray(q, dtype=np.float64)
    B, S, Hq, D = q.shape
    Hkv = np.asarray(k_cache).shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    g = Hq // Hkv
    p = _prefix(prefix, B)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, S, Hq, D), dtype=np.float64)
    for b in range(B):
        T = int(p[b]) + S
        kl = gather_logical(k_cache, kv_map, b, T).astype(np.float64)
        vl = gather_logical(v_cache, kv_map, b, T).astype(np.float64)
        qr = rope_rotate(q[b], p[b] + np.arange(S), rope_theta)
        kr = rope_rotate(kl, np.arange(T), rope_theta)
        for h in range(Hq):
            kv = h // g
            pr = _prefix_probs((qr[:, h, :] @ kr[:, kv, :].T) * scale, int(p[b]))
            out[b, :, h, :] = pr @ vl[:, kv, :]
    return out


def attention_i16_cached(q, k_cache, v_cache, kv_map, prefix=None, rope_theta=10000.0, score_scale=1.0):
    """Cached prefill of the int16 variant: integer RoPE of Q (position
    P_b + i) and of the cached K (position j), exact int32 scores, fp64
    softmax and P.V."""
    q = np.asarray(q, dtype=np.int64)
    B, S, Hq, D = q.shape
    Hkv = np.asarray(k_cache).shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    g = Hq // Hkv
    p = _prefix(prefix, B)
    table = rope_table_q14(int(p.max()) + S, D, rope_theta)
    out = np.zeros((B, S, Hq, D), dtype=np.float64)
    for b in range(B):
        T = int(p[b]) + S
        kl = gather_logical(k_cache, kv_map, b, T).astype(np.int64)
        vl = gather_logical(v_cache, kv_map, b, T).astype(np.float64)
        qr = rope_rotate_i16(q[b], p[b] + np.arange(S), rope_theta, table)
        kr = rope_rotate_i16(kl, np.arange(T), rope_theta, table)
        for h in range(Hq):
            kv = h // g
            s = scores_i32(qr[:, h, :], kr[:, kv, :])
            pr = _prefix_probs(s.astype(np.float64) * float(score_scale), int(p[b]))
            out[b, :, h, :] = pr @ vl[:, kv, :]
    return out


def attention_cached_rows(q, k_cache, v_cache, kv_map, rows, prefix=None, rope_theta=10000.0, scale=None):
    """:func:`attention_cached` for selected output rows (b, h, i) only."""
    q = np.asarray(q)
    B, S, Hq, D = q.shape
    Hkv = np.asarray(k_cache).shape[1]
    g = Hq // Hkv
    p = _prefix(prefix, B)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rows = list(rows)
    out = np.zeros((len(rows), D), dtype=np.float64)
    for n, (b, h, i) in enumerate(rows):
        kv = h // g
        T = int(p[b]) + i + 1
        kl = gather_logical(k_cache, kv_map, b, T)[:, kv:kv + 1, :].astype(np.float64)
        vl = gather_logical(v_cache, kv_map, b, T)[:, kv, :].astype(np.float64)
        qi = rope_rotate(np.asarray(q[b, i:i + 1, h:h + 1, :], dtype=np.float64), [p[b] + i], rope_theta)[0, 0]
        kk = rope_rotate(kl, np.arange(T), rope_theta)[:, 0]
        sc = (kk @ qi) * scale
        e = np.exp(sc - sc.max())
        out[n] = (e @ vl) / e.sum()
    return out
