"""Pins the CPU oracle to facts outside itself (no GPU involved).

Each test checks the oracle against something the pages or the mathematics
fix: closed forms, invariants of RoPE and softmax, a library routine on an
independently rotated input, 50-digit brute force, hand-derived fixed-point
values.  A plausible slip anywhere in the oracle (a dropped term, a sign, a
pair index, a transposed operand, the GQA head map) fails at least one.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden

mpmath = pytest.importorskip("mpmath")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _complex_rotate(x, positions, theta):
    """Independent RoPE: pairs as complex numbers times e^{i p theta_k}."""
    D = x.shape[-1]
    inv = np.float64(theta) ** (-np.arange(0, D, 2, dtype=np.float64) / D)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    zr = z * np.exp(1j * ang)[:, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = zr.real
    out[..., 1::2] = zr.imag
    return out


# ---------------------------------------------------------------- RoPE pins

def test_rope_preserves_pair_norms():
    x = _rand((40, 3, 64), 1)
    pos = np.arange(40) * 37 + 5
    r = oracle.rope_rotate(x, pos, 1e4)
    n0 = np.hypot(x[..., 0::2], x[..., 1::2])
    n1 = np.hypot(r[..., 0::2], r[..., 1::2])
    np.testing.assert_allclose(n1, n0, rtol=1e-14, atol=0)


def test_rope_matches_complex_multiply():
    for D, theta in [(64, 1e4), (96, 1e4), (128, 1e6), (8, 500.0)]:
        x = _rand((33, 2, D), D)
        pos = np.arange(33) * 11 + 3
        np.testing.assert_allclose(oracle.rope_rotate(x, pos, theta), _complex_rotate(x, pos, theta),
                                   rtol=0, atol=1e-12)


def test_rope_position_zero_is_identity():
    x = _rand((1, 4, 96), 2)
    assert np.array_equal(oracle.rope_rotate(x, [0], 1e4), x)


def test_rope_pair_layout_is_interleaved():
    # only the pair (X[2k], X[2k+1]) mixes: a unit vector in slot 2k stays in slots 2k, 2k+1
    D = 16
    for k in range(D // 2):
        x = np.zeros((1, 1, D))
        x[0, 0, 2 * k] = 1.0
        r = oracle.rope_rotate(x, [3], 1e4)[0, 0]
        a = 3 * 1e4 ** (-2 * k / D)
        expect = np.zeros(D)
        expect[2 * k] = math.cos(a)
        expect[2 * k + 1] = math.sin(a)
        np.testing.assert_allclose(r, expect, atol=1e-15)


def test_rope_scores_depend_only_on_relative_position():
    D = 64
    q = _rand((24, 1, D), 3)
    k = _rand((24, 1, D), 4)
    pos = np.arange(24)
    for shift in (1, 100, 3000):
        s0 = oracle.rope_rotate(q, pos, 1e4)[:, 0] @ oracle.rope_rotate(k, pos, 1e4)[:, 0].T
        s1 = oracle.rope_rotate(q, pos + shift, 1e4)[:, 0] @ oracle.rope_rotate(k, pos + shift, 1e4)[:, 0].T
        np.testing.assert_allclose(s1, s0, rtol=0, atol=1e-11)


# ------------------------------------------------------------- softmax pins

def test_causal_probs_rows_sum_to_one_and_mask_is_exact_zero():
    sc = _rand((50, 50), 5) * 6.0
    p = oracle.causal_probs(sc)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p[np.triu_indices(50, 1)] == 0.0)
    assert np.all(p[np.tril_indices(50)] > 0.0)
    assert p[0, 0] == 1.0


# ----------------------------------------------------------- attention pins

def test_closed_form_two_tokens():
    g = {r[0]: float(r[1]) for r in read_golden("closed_form_s2_d2.txt")}
    q = np.zeros((1, 2, 1, 2))
    q[..., 0] = 1.0
    v = np.zeros((1, 2, 1, 2))
    v[0, 0, 0, 0] = 1.0
    v[0, 1, 0, 1] = 1.0
    o = oracle.attention(q, q.copy(), v, rope_theta=1e4)
    np.testing.assert_array_equal(o[0, 0, 0], [1.0, 0.0])
    np.testing.assert_allclose(o[0, 1, 0], [g["P10"], g["P11"]], rtol=0, atol=1e-12)
    # the scores themselves, through the softmax-free path
    qr = oracle.rope_rotate(q[0], [0, 1], 1e4)[:, 0]
    s = qr @ qr.T / math.sqrt(2)
    np.testing.assert_allclose([s[1, 0], s[1, 1]], [g["s10"], g["s11"]], rtol=0, atol=1e-12)


def test_first_output_row_is_first_value_row_exactly():
    B, S, Hq, Hkv, D = 2, 9, 4, 2, 32
    q, k, v = _rand((B, S, Hq, D), 6), _rand((B, S, Hkv, D), 7), _rand((B, S, Hkv, D), 8)
    o = oracle.attention(q, k, v, pos_offsets=[0, 17])
    for h in range(Hq):
        assert np.array_equal(o[:, 0, h], v[:, 0, h // 2])


def _sdpa_reference(q, k, v, pos_offsets, theta, scale):
    """torch SDPA (fp64, CPU) on independently rotated inputs; GQA by repeat."""
    B, S, Hq, D = q.shape
    g = Hq // k.shape[2]
    out = np.zeros_like(q)
    for b in range(B):
        pos = pos_offsets[b] + np.arange(S)
        qr = torch.from_numpy(_complex_rotate(q[b], pos, theta)).permute(1, 0, 2)
        kr = torch.from_numpy(_complex_rotate(k[b], pos, theta)).permute(1, 0, 2)
        vv = torch.from_numpy(v[b]).permute(1, 0, 2)
        kr = kr.repeat_interleave(g, dim=0)
        vv = vv.repeat_interleave(g, dim=0)
        o = torch.nn.functional.scaled_dot_product_attention(qr, kr, vv, is_causal=True, scale=scale)
        out[b] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("B,S,Hq,Hkv,D,theta", [
    (1, 32, 1, 1, 64, 1e4),
    (2, 45, 4, 2, 96, 1e4),
    (1, 70, 4, 1, 128, 1e6),
])
def test_matches_library_sdpa_on_independent_rotation(B, S, Hq, Hkv, D, theta):
    q = _rand((B, S, Hq, D), 10) * 1.7
    k = _rand((B, S, Hkv, D), 11) * 1.3
    v = _rand((B, S, Hkv, D), 12)
    off = [0, 123][:B]
    o = oracle.attention(q, k, v, pos_offsets=off, rope_theta=theta)
    ref = _sdpa_reference(q, k, v, off, theta, 1.0 / math.sqrt(D))
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def _mp_attention(q, k, v, offs, theta, scale):
    """50-digit brute force of RoPE causal attention, written from scratch."""
    mp = mpmath.mp
    B, S, Hq, D = q.shape
    g = Hq // k.shape[2]
    out = np.zeros(q.shape)
    for b in range(B):
        for h in range(Hq):
            kv = h // g

            def rot(x, p):
                r = []
                for kk in range(D // 2):
                    ang = mp.mpf(p) * mp.power(mp.mpf(theta), mp.mpf(-2 * kk) / D)
                    c, s = mp.cos(ang), mp.sin(ang)
                    a, bb = mp.mpf(x[2 * kk]), mp.mpf(x[2 * kk + 1])
                    r += [a * c - bb * s, a * s + bb * c]
                return r

            qs = [rot(q[b, i, h], offs[b] + i) for i in range(S)]
            ks = [rot(k[b, j, kv], offs[b] + j) for j in range(S)]
            for i in range(S):
                sc = [mp.fsum(qs[i][d] * ks[j][d] for d in range(D)) * scale for j in range(i + 1)]
                m = max(sc)
                e = [mp.exp(x - m) for x in sc]
                l = mp.fsum(e)
                for d in range(D):
                    out[b, i, h, d] = float(mp.fsum(e[j] * mp.mpf(v[b, j, kv, d]) for j in range(i + 1)) / l)
    return out


def test_brute_force_50_digits():
    mpmath.mp.dps = 50
    B, S, Hq, Hkv, D = 2, 6, 4, 2, 8
    q = _rand((B, S, Hq, D), 20) * 2.0
    k = _rand((B, S, Hkv, D), 21) * 2.0
    v = _rand((B, S, Hkv, D), 22)
    offs = [0, 5]
    o = oracle.attention(q, k, v, pos_offsets=offs, rope_theta=1e4)
    ref = _mp_attention(q, k, v, offs, 1e4, mpmath.mpf(1) / mpmath.sqrt(D))
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    B, S, Hq, Hkv, D = 1, 20, 6, 2, 16
    q, k, v = _rand((B, S, Hq, D), 30), _rand((B, S, Hkv, D), 31), _rand((B, S, Hkv, D), 32)
    o = oracle.attention(q, k, v)
    o2 = oracle.attention(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2))
    assert np.array_equal(o, o2)


def test_offsets_do_not_change_the_output():
    B, S, Hq, Hkv, D = 3, 25, 2, 2, 32
    q, k, v = _rand((B, S, Hq, D), 40), _rand((B, S, Hkv, D), 41), _rand((B, S, Hkv, D), 42)
    o0 = oracle.attention(q, k, v, pos_offsets=[0, 0, 0])
    o1 = oracle.attention(q, k, v, pos_offsets=[7, 1000, 4000])
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-11)
    # but the rotation itself does move: different offsets give different Q'
    assert not np.allclose(oracle.rope_rotate(q[0], np.arange(S), 1e4),
                           oracle.rope_rotate(q[0], np.arange(S) + 7, 1e4))


def test_rows_match_full_attention():
    B, S, Hq, Hkv, D = 2, 40, 4, 2, 32
    q, k, v = _rand((B, S, Hq, D), 50), _rand((B, S, Hkv, D), 51), _rand((B, S, Hkv, D), 52)
    offs = [3, 50]
    o = oracle.attention(q, k, v, pos_offsets=offs)
    rows = [(0, 0, 0), (0, 3, 39), (1, 1, 17), (1, 2, 1)]
    r = oracle.attention_rows(q, k, v, rows, pos_offsets=offs)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(r[n], o[b, i, h], rtol=0, atol=1e-13)


# ---------------------------------------------------------- int16 pins

def test_int16_worked_values():
    inv = oracle.rope_inv_freq(2, 1e4)
    assert inv[0] == 1.0
    C, S = oracle.rope_table_q14(2, 2, 1e4)
    assert (C[0, 0], S[0, 0]) == (16384, 0)
    for p, kk, c, s, x, y, xr, yr in (map(int, r) for r in read_golden("int16_rope_worked.txt")):
        assert (C[p, kk], S[p, kk]) == (c, s)
        r = oracle.rope_rotate_i16(np.array([[[x, y]]]), [p], 1e4)
        assert (r[0, 0, 0], r[0, 0, 1]) == (xr, yr)


def test_int16_position_zero_is_identity_for_every_input():
    x = np.arange(-2048, 2048, dtype=np.int64)
    assert np.array_equal((x * 16384 + 8192) >> 14, x)
    xx = np.stack([x, x[::-1]], axis=-1).reshape(4096, 1, 2)
    assert np.array_equal(oracle.rope_rotate_i16(xx, np.zeros(4096, dtype=np.int64), 1e4), xx)


def test_int16_table_matches_50_digit_rounding():
    mpmath.mp.dps = 50
    D, theta = 128, 1e4
    C, S = oracle.rope_table_q14(2048, D, theta)
    inv = [float(theta) ** (-2.0 * k / D) for k in range(D // 2)]
    rng = np.random.default_rng(60)
    for p, k in zip(rng.integers(0, 2048, 400), rng.integers(0, D // 2, 400)):
        a = mpmath.mpf(float(p) * inv[k])     # the fp64 angle, evaluated exactly
        for val, got in ((mpmath.cos(a), C[p, k]), (mpmath.sin(a), S[p, k])):
            x = val * 16384
            want = int(mpmath.floor(abs(x) + mpmath.mpf("0.5"))) * (1 if x >= 0 else -1)
            assert got == want
    assert np.abs(C).max() == 16384 and np.abs(S).max() <= 16384


def test_int16_rotation_tracks_float_rotation():
    # integer RoPE = float RoPE within table rounding (<= 0.5*(|x|+|y|)/2^14 <= 0.125)
    # plus the final round-half-up (<= 0.5)
    rng = np.random.default_rng(61)
    x = rng.integers(-2048, 2048, size=(300, 2, 64))
    pos = rng.integers(0, 4096, size=300)
    ri = oracle.rope_rotate_i16(x, pos, 1e4)
    rf = oracle.rope_rotate(x.astype(np.float64), pos, 1e4)
    assert np.abs(ri - rf).max() <= 0.625 + 1e-9


def test_int16_rotated_range_bound():
    C, S = oracle.rope_table_q14(2048, 128, 1e4)
    worst = 0
    for x in (-2048, 2047):
        for y in (-2048, 2047):
            worst = max(worst, np.abs((x * C - y * S + 8192) >> 14).max(),
                        np.abs((x * S + y * C + 8192) >> 14).max())
    assert worst <= 2897
    assert 128 * 2897 ** 2 < 2 ** 31


def test_int16_scores_exact_against_int64_brute_force():
    rng = np.random.default_rng(62)
    q = rng.integers(-2897, 2898, size=(19, 128))
    k = rng.integers(-2897, 2898, size=(23, 128))
    s = oracle.scores_i32(q, k)
    brute = np.array([[sum(int(a) * int(b) for a, b in zip(qi, kj)) for kj in k] for qi in q])
    assert np.array_equal(s, brute)
    extreme = np.full((1, 128), 2897)
    assert oracle.scores_i32(extreme, -extreme)[0, 0] == -128 * 2897 ** 2


def test_int16_attention_matches_sdpa_on_integer_scores():
    rng = np.random.default_rng(63)
    B, S, H, D = 1, 37, 2, 64
    q = rng.integers(-2048, 2048, size=(B, S, H, D))
    k = rng.integers(-2048, 2048, size=(B, S, H, D))
    v = rng.standard_normal((B, S, H, D))
    scale = 2.0 ** -22 / 8.0
    o = oracle.attention_i16(q, k, v, rope_theta=1e4, score_scale=scale)
    pos = np.arange(S)
    for h in range(H):
        qr = torch.from_numpy(oracle.rope_rotate_i16(q[0], pos, 1e4)[:, h].astype(np.float64))
        kr = torch.from_numpy(oracle.rope_rotate_i16(k[0], pos, 1e4)[:, h].astype(np.float64))
        ref = torch.nn.functional.scaled_dot_product_attention(
            qr[None], kr[None], torch.from_numpy(v[0, :, h])[None], is_causal=True, scale=scale)[0]
        np.testing.assert_allclose(o[0, :, h], ref.numpy(), rtol=0, atol=1e-12)
    assert np.array_equal(o[0, 0], v[0, 0])


def test_int16_rows_match_full():
    rng = np.random.default_rng(64)
    B, S, Hq, Hkv, D = 2, 30, 4, 2, 32
    q = rng.integers(-2048, 2048, size=(B, S, Hq, D))
    k = rng.integers(-2048, 2048, size=(B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    offs = [0, 9]
    o = oracle.attention_i16(q, k, v, pos_offsets=offs, score_scale=1e-6)
    rows = [(0, 0, 0), (1, 3, 29), (0, 2, 11)]
    r = oracle.attention_i16_rows(q, k, v, rows, pos_offsets=offs, score_scale=1e-6)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(r[n], o[b, i, h], rtol=0, atol=1e-13)
