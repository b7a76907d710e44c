"""Pins the per-token int16 quantisation part of the CPU oracle (no GPU).

Worked codes (including a round-half-to-even case), the invariants of the
per-row scale, the reduction to the already-pinned int16 attention when the
inputs are their own codes, and closeness to the fp64 float attention.
"""

import numpy as np

import oracle


def test_worked_codes():
    # absmax 1 -> scale 2047: 0.5 * 2047 = 1023.5 -> 1024 (even), 0.25 * 2047 = 511.75 -> 512
    codes, inv = oracle.quantize_rows_i16(np.array([[0.5, -1.0, 0.25, 0.0]], dtype=np.float32))
    assert codes.tolist() == [[1024, -2047, 512, 0]]
    assert inv[0] == 1.0 / 2047


def test_round_half_to_even():
    # absmax 2047/1024 -> scale exactly 1024; 1022.5 and 1021.5 both go to 1022, -0.5 to 0
    row = np.array([[2047 / 1024, 1022.5 / 1024, 1021.5 / 1024, -0.5 / 1024]], dtype=np.float32)
    codes, _ = oracle.quantize_rows_i16(row)
    assert codes.tolist() == [[2047, 1022, 1022, 0]]


def test_zero_row():
    codes, inv = oracle.quantize_rows_i16(np.zeros((2, 3, 8), dtype=np.float32))
    assert not codes.any() and not inv.any()


def test_scale_is_per_row_and_round_trip_is_within_half_a_step():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((5, 7, 64)) * rng.uniform(0.01, 100.0, (5, 7, 1))).astype(np.float32)
    codes, inv = oracle.quantize_rows_i16(x)
    assert (np.abs(codes).max(axis=-1) == 2047).all()
    err = np.abs(codes * inv[..., None] - x.astype(np.float64))
    assert (err <= inv[..., None] * (0.5 + 1e-6)).all()


def test_integer_rows_at_full_range_reduce_to_the_int16_path():
    """Rows whose absmax is 2047 are their own codes (scale 1, factor 1), so the
    quantised attention is the int16 attention with the same score scale."""
    rng = np.random.default_rng(11)
    B, S, Hq, Hkv, D = 1, 20, 4, 2, 16
    q = rng.integers(-2047, 2048, (B, S, Hq, D))
    k = rng.integers(-2047, 2048, (B, S, Hkv, D))
    q[..., 0] = 2047
    k[..., 3] = -2047
    v = rng.standard_normal((B, S, Hkv, D))
    scale = 2.0 ** -22
    a = oracle.attention_i16_quantized(q.astype(np.float32), k.astype(np.float32), v, rope_theta=1e4,
                                       score_scale=scale)
    b = oracle.attention_i16(q, k, v, rope_theta=1e4, score_scale=scale)  # both factors are 2047 / 2047
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-15)


def test_quantised_attention_tracks_float_attention():
    rng = np.random.default_rng(21)
    B, S, Hq, Hkv, D = 2, 40, 4, 2, 64
    q = rng.standard_normal((B, S, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, S, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((B, S, Hkv, D))
    exact = oracle.attention(q, k, v, pos_offsets=[0, 9], rope_theta=1e4)
    quant = oracle.attention_i16_quantized(q, k, v, pos_offsets=[0, 9], rope_theta=1e4)
    err = np.abs(quant - exact)
    # 12-bit codes: relative score error ~ 1e-3, far inside the bf16 bar and not zero
    assert 0 < err.max() <= 1e-2 and err.mean() <= 1e-3


def test_rows_match_full():
    rng = np.random.default_rng(5)
    B, S, Hq, Hkv, D = 1, 30, 2, 1, 32
    q = rng.standard_normal((B, S, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, S, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((B, S, Hkv, D))
    full = oracle.attention_i16_quantized(q, k, v, pos_offsets=[4], rope_theta=1e4)
    rows = [(0, 0, 0), (0, 1, 17), (0, 0, 29)]
    got = oracle.attention_i16_quantized_rows(q, k, v, rows, pos_offsets=[4], rope_theta=1e4)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(got[n], full[b, i, h], rtol=0, atol=1e-14)
