"""Pins the KV-cache part of the CPU oracle (no GPU involved).

The cached prefill must reach, row for row, what a plain causal prefill of
the whole sequence gives (the chunks only change where the keys come from);
the index maps and the cache update are fixed by their definitions on small
worked examples; a 50-digit brute force written from scratch checks one
scattered-cache case end to end.
"""

import math

import numpy as np
import pytest

import oracle

mpmath = pytest.importorskip("mpmath")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _int(shape, seed, lim=2048):
    return np.random.default_rng(seed).integers(-lim, lim, size=shape)


# ------------------------------------------------------------ index maps

def test_ring_map_wraps_at_the_ring_size():
    # 128 slots starting at 120: 120..127, then 0.. (the bit-mask ring of the
    # 2kiu.com page, §3.4: index & 0x7F).
    got = oracle.ring_index_map(128, 120, 12)
    assert got.tolist() == [120, 121, 122, 123, 124, 125, 126, 127, 0, 1, 2, 3]
    assert oracle.ring_index_map(8, 0, 3).tolist() == [0, 1, 2]


def test_paged_map_worked_example():
    # Logical blocks 0, 1, 2 of 4 slots live in physical blocks 3, 0, 2.
    got = oracle.paged_index_map([3, 0, 2], 4, 10)
    assert got.tolist() == [12, 13, 14, 15, 0, 1, 2, 3, 8, 9]


# ------------------------------------------------------------ cache update

def test_update_writes_exactly_the_new_slots():
    n_slots, Hkv, D = 20, 2, 4
    kc = _rand((n_slots, Hkv, D), 1)
    vc = _rand((n_slots, Hkv, D), 2)
    kn = _rand((2, 3, Hkv, D), 3)
    vn = _rand((2, 3, Hkv, D), 4)
    kv_map = np.array([[5, 6, 7, 8, 9, 0, 0], [19, 18, 1, 2, 3, 4, 0]])
    prefix = [2, 3]
    k2, v2 = oracle.kv_cache_update(kc, vc, kn, vn, kv_map, prefix)
    new_slots = {7: (0, 0), 8: (0, 1), 9: (0, 2), 2: (1, 0), 3: (1, 1), 4: (1, 2)}
    for s in range(n_slots):
        if s in new_slots:
            b, i = new_slots[s]
            assert np.array_equal(k2[s], kn[b, i]) and np.array_equal(v2[s], vn[b, i])
        else:
            assert np.array_equal(k2[s], kc[s]) and np.array_equal(v2[s], vc[s])
    # the inputs are not modified
    assert not np.array_equal(k2, kc)


def test_update_rejects_colliding_slots():
    kc = np.zeros((8, 1, 2))
    with pytest.raises(ValueError):
        oracle.kv_cache_update(kc, kc, np.ones((2, 1, 1, 2)), np.ones((2, 1, 1, 2)), [[3], [3]], [0, 0])


# ------------------------------------------------------------ cached prefill

def _pool(seqs, n_slots, maps, Hkv, D):
    """Scatter each sequence's logical K (or V) [T_b][Hkv][D] into a pool."""
    pool = _rand((n_slots, Hkv, D), 99) * 50.0  # garbage in unused slots
    for b, x in enumerate(seqs):
        for j in range(x.shape[0]):
            pool[maps[b][j]] = x[j]
    return pool


@pytest.mark.parametrize("Hq,Hkv,D", [(2, 2, 8), (4, 2, 16)])
def test_cached_rows_equal_full_prefill_rows(Hq, Hkv, D):
    """Chunk [P_b, P_b + S) of sequence b, read through a scattered cache,
    equals rows P_b.. of one causal prefill of the whole sequence."""
    S, prefix, theta = 5, [0, 4, 11], 1e4
    B = len(prefix)
    full = [(_rand((1, p + S, Hq, D), 10 + b), _rand((1, p + S, Hkv, D), 20 + b), _rand((1, p + S, Hkv, D), 30 + b))
            for b, p in enumerate(prefix)]
    n_slots = 64
    perm = np.random.default_rng(5).permutation(n_slots)
    width = max(prefix) + S
    maps, start = [], 0
    for p in prefix:
        maps.append(list(perm[start:start + p + S]) + [0] * (width - p - S))  # padding is never read
        start += p + S
    kv_map = np.array(maps)
    kc = _pool([f[1][0] for f in full], n_slots, maps, Hkv, D)
    vc = _pool([f[2][0] for f in full], n_slots, maps, Hkv, D)
    q = np.stack([full[b][0][0, p:p + S] for b, p in enumerate(prefix)])
    got = oracle.attention_cached(q, kc, vc, kv_map, prefix, rope_theta=theta)
    for b, p in enumerate(prefix):
        want = oracle.attention(*full[b], rope_theta=theta)[0, p:p + S]
        np.testing.assert_allclose(got[b], want, rtol=0, atol=1e-12)


def test_cached_result_does_not_depend_on_slot_placement():
    Hq, Hkv, D, S, P = 4, 1, 8, 6, 9
    k = _rand((P + S, Hkv, D), 1)
    v = _rand((P + S, Hkv, D), 2)
    q = _rand((1, S, Hq, D), 3)
    ident = np.arange(P + S)[None, :]
    a = oracle.attention_cached(q, k, v, ident, [P])
    ring = oracle.ring_index_map(16, 13, P + S)
    kr = np.zeros((16, Hkv, D))
    vr = np.zeros((16, Hkv, D))
    kr[ring] = k
    vr[ring] = v
    b = oracle.attention_cached(q, kr, vr, ring[None, :], [P])
    assert np.array_equal(a, b)


def test_chunked_prefill_pipeline_matches_one_prefill():
    """Chunks of 5, 7 and 4 tokens through kv_cache_update + attention_cached
    on a wrapped ring equal the single causal prefill of all 16 tokens."""
    Hq, Hkv, D, theta = 4, 2, 16, 5e5
    T = 16
    q = _rand((1, T, Hq, D), 40)
    k = _rand((1, T, Hkv, D), 41)
    v = _rand((1, T, Hkv, D), 42)
    want = oracle.attention(q, k, v, rope_theta=theta)
    ring = oracle.ring_index_map(32, 25, T)[None, :]
    kc = np.full((32, Hkv, D), np.nan)
    vc = np.full((32, Hkv, D), np.nan)
    pos, outs = 0, []
    for n in (5, 7, 4):
        kc, vc = oracle.kv_cache_update(kc, vc, k[:, pos:pos + n], v[:, pos:pos + n], ring, [pos])
        outs.append(oracle.attention_cached(q[:, pos:pos + n], kc, vc, ring, [pos], rope_theta=theta))
        pos += n
    np.testing.assert_allclose(np.concatenate(outs, axis=1), want, rtol=0, atol=1e-12)


def test_cached_rows_match_cached():
    Hq, Hkv, D, S = 4, 2, 8, 7
    prefix = [3, 0]
    kc = _rand((40, Hkv, D), 7)
    vc = _rand((40, Hkv, D), 8)
    kv_map = np.stack([np.arange(10), 39 - np.arange(10)])
    q = _rand((2, S, Hq, D), 9)
    full = oracle.attention_cached(q, kc, vc, kv_map, prefix)
    rows = [(0, 1, 0), (0, 3, 6), (1, 0, 0), (1, 2, 4)]
    got = oracle.attention_cached_rows(q, kc, vc, kv_map, rows, prefix)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(got[n], full[b, i, h], rtol=0, atol=1e-13)


def test_cached_brute_force_50_digits():
    """Scattered cache, prefix 3, two new tokens: every quantity in 50 digits."""
    mp = mpmath.mp
    mp.dps = 50
    Hq, Hkv, D, S, P, theta = 2, 1, 4, 2, 3, 1e4
    kc = _rand((9, Hkv, D), 61) * 2.0
    vc = _rand((9, Hkv, D), 62)
    q = _rand((1, S, Hq, D), 63) * 2.0
    slots = [7, 2, 5, 0, 8]  # logical 0..4
    got = oracle.attention_cached(q, kc, vc, np.array([slots]), [P], rope_theta=theta)

    def rot(x, p):
        r = []
        for kk in range(D // 2):
            ang = mp.mpf(p) * mp.power(mp.mpf(theta), mp.mpf(-2 * kk) / D)
            a, b = mp.mpf(x[2 * kk]), mp.mpf(x[2 * kk + 1])
            r += [a * mp.cos(ang) - b * mp.sin(ang), a * mp.sin(ang) + b * mp.cos(ang)]
        return r

    for h in range(Hq):
        for i in range(S):
            qi = rot(q[0, i, h], P + i)
            sc = []
            for j in range(P + i + 1):
                kj = rot(kc[slots[j], 0], j)
                sc.append(mp.fsum(qi[d] * kj[d] for d in range(D)) / mp.sqrt(D))
            m = max(sc)
            e = [mp.exp(x - m) for x in sc]
            for d in range(D):
                ref = mp.fsum(e[j] * mp.mpf(vc[slots[j], 0, d]) for j in range(P + i + 1)) / mp.fsum(e)
                assert abs(got[0, i, h, d] - float(ref)) < 1e-13


def test_int16_cached_equals_full_prefill_rows():
    Hq, Hkv, D, S, P, theta = 4, 2, 16, 6, 10, 1e4
    scale = 2.0 ** -22 / 4.0
    q = _int((1, P + S, Hq, D), 70)
    k = _int((1, P + S, Hkv, D), 71)
    v = _rand((1, P + S, Hkv, D), 72)
    want = oracle.attention_i16(q, k, v, rope_theta=theta, score_scale=scale)[0, P:]
    ring = oracle.ring_index_map(32, 20, P + S)
    kc = np.zeros((32, Hkv, D), dtype=np.int64)
    vc = np.zeros((32, Hkv, D))
    kc[ring] = k[0]
    vc[ring] = v[0]
    got = oracle.attention_i16_cached(q[:, P:], kc, vc, ring[None, :], [P], rope_theta=theta, score_scale=scale)
    np.testing.assert_allclose(got[0], want, rtol=0, atol=1e-13)
