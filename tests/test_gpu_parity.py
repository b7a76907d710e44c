"""GPU parity: the HIP path (through the C-ABI) against the fp64 CPU oracle.

Small cases compare every element; full-size workloads compare sampled output
rows (each computed by the oracle one at a time) plus whole heads.  Floating
tolerances: fp32 inputs max-abs 1e-5; bf16 inputs and the int16 variant's
output max-abs 1e-2 and mean-abs 1e-3.  The int16 rotation and int32 scores are
compared bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
import rope_causal_attention_amd as pa
import synth
from gpu_common import (announce, assert_close, need_gpu, oracle_full, run_gpu,
                        to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


# ------------------------------------------------------------ float, whole O

SMALL_CASES = [
    # name, batch, Hq, Hkv, S, D, dtype, theta, offsets
    ("tiny_f32", 1, 1, 1, 32, 64, "f32", 1e4, None),
    ("f32_ragged_d96_gqa", 2, 4, 2, 77, 96, "f32", 1e4, [0, 5]),
    ("f32_d128_2blocks", 1, 2, 1, 200, 128, "f32", 1e6, None),
    ("bf16_d64_ragged", 2, 3, 3, 301, 64, "bf16", 1e4, [0, 17]),
    ("bf16_d96_ragged", 1, 4, 2, 333, 96, "bf16", 1e4, None),
    ("bf16_d128_ragged", 1, 2, 2, 390, 128, "bf16", 1e6, [100]),
    ("bf16_d128_s1", 3, 2, 1, 1, 128, "bf16", 1e4, None),
    ("bf16_d96_s33", 1, 2, 2, 33, 96, "bf16", 1e4, None),
    ("bf16_d64_s129", 1, 8, 8, 129, 64, "bf16", 1e4, None),
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_float_small_full_compare(case):
    name, B, Hq, Hkv, S, D, dt, theta, offs = case
    announce(name)
    max_seq = S + (max(offs) if offs else 0)
    w = synth.Workload(name, B, Hq, Hkv, S, D, dt, theta, seed=sum(map(ord, name)), max_seq=max_seq)
    q, k, v = synth.make_inputs(w)
    got = run_gpu(w, q, k, v, pos_offsets=offs)
    want = oracle_full(w, q, k, v, pos_offsets=offs)
    mx, mean = assert_close(got.numpy(), want, dt)
    announce(name, f"max {mx:.2e} mean {mean:.2e}")


# Shapes with at least 256 workgroups of 256 query rows run the eight-wave
# ping-pong kernel; the cases above run the four-wave kernel.
PINGPONG_CASES = [
    # name, batch, Hq, Hkv, S, D, theta, offsets
    ("pp_d96_ragged_gqa", 2, 32, 16, 1100, 96, 1e4, [0, 37]),
    ("pp_d128_ragged", 2, 32, 32, 1030, 128, 1e6, None),
    ("pp_d64_exact", 1, 64, 8, 1024, 64, 1e4, [5]),
    ("pp_d128_gqa4_offsets", 2, 32, 8, 1100, 128, 1e4, [0, 300]),  # two-group schedule, GQA 4, offsets
    # Paired launches (224..256 pairs of query blocks on a 256-CU device): each
    # workgroup runs block n-1-j, then block j of the same head.
    ("paired_d96_odd_ragged", 1, 64, 16, 1700, 96, 1e4, [3]),  # 7 blocks: the middle one runs alone
    ("paired_d128_last_block_8_rows", 2, 32, 8, 1800, 128, 1e6, [0, 77]),  # 8 blocks, the last holds 8 rows
    ("paired_d64_exact", 1, 64, 64, 2048, 64, 1e4, None),
    # (batch, head) counts that are not a multiple of 8 take the plain
    # round-robin order instead of per-XCD head ranges.
    ("paired_bh60_gqa5_d64", 1, 60, 12, 2048, 64, 1e4, [11]),  # 240 pairs
    ("pp_bh36_gqa3_d96", 1, 36, 12, 2000, 96, 1e4, None),  # 288 blocks, unpaired
]


@pytest.mark.parametrize("case", PINGPONG_CASES, ids=[c[0] for c in PINGPONG_CASES])
def test_pingpong_shapes_full_compare(case):
    name, B, Hq, Hkv, S, D, theta, offs = case
    n_qb = (S + 255) // 256
    assert B * Hq * n_qb >= 256
    if name.startswith("paired"):
        assert 224 <= (n_qb + 1) // 2 * B * Hq <= 256
    announce(name)
    max_seq = S + (max(offs) if offs else 0)
    w = synth.Workload(name, B, Hq, Hkv, S, D, "bf16", theta, seed=sum(map(ord, name)), max_seq=max_seq)
    q, k, v = synth.make_inputs(w)
    got = run_gpu(w, q, k, v, pos_offsets=offs)
    want = oracle_full(w, q, k, v, pos_offsets=offs)
    mx, mean = assert_close(got.numpy(), want, "bf16")
    announce(name, f"max {mx:.2e} mean {mean:.2e}")


def test_tiny_workload_exact_config():
    w = synth.WORKLOADS["tiny_f32_s32_d64"]
    announce(w.name)
    q, k, v = synth.make_inputs(w)
    got = run_gpu(w, q, k, v)
    want = oracle_full(w, q, k, v)
    assert_close(got.numpy(), want, "f32")


@pytest.mark.parametrize("name", ["mha_bf16_h32_s512_d128", "gqa_bf16_b16_h16kv8_s512_d128"])
def test_full_workload_whole_output(name):
    w = synth.WORKLOADS[name]
    announce(name)
    q, k, v = synth.make_inputs(w)
    got = run_gpu(w, q, k, v)
    want = oracle_full(w, q, k, v)
    mx, mean = assert_close(got.numpy(), want, w.dtype)
    announce("margin", name, f"max {mx:.3e} mean {mean:.3e}")


@pytest.mark.parametrize("reading", ["independent", "shared"])
def test_long_prompt_workload(reading):
    """seq 4096, D 96, per-head scales: the whole O (all 32 heads) against the oracle."""
    w = synth.workload("mha_bf16_h32_s4096_d96", head_scale=reading)
    announce(w.name, reading)
    q, k, v = synth.make_inputs(w)
    got = run_gpu(w, q, k, v).numpy()
    want = oracle_full(w, q, k, v)
    mx, mean = assert_close(got, want, "bf16")
    announce("margin", w.name, reading, f"max {mx:.3e} mean {mean:.3e}")


# ------------------------------------------------------------ int16 variant

def _i16_handle(w, max_seq=None):
    return pa.PrefillAttention(w.n_heads, w.n_kv_heads, w.head_dim, max_seq or w.seq_len, w.rope_theta)


UNWRITTEN = -2 ** 31  # score-export buffers start filled with this


def _score_buffer(B, H, S):
    return torch.full((B, H, S, S), UNWRITTEN, dtype=torch.int32, device="cuda")


def _assert_causal_scores(got, want, what):
    """got: the export's [S][S] block; want: the oracle's full [S][S] scores.
    Keys at or before the query bit-equal, the rest left unwritten."""
    got = got.cpu().numpy().astype(np.int64)
    low = np.tril(np.ones(got.shape, dtype=bool))
    bad = np.count_nonzero(got[low] != want[low])
    assert bad == 0, f"{what}: {bad} mismatching causal scores"
    assert np.all(got[~low] == UNWRITTEN), f"{what}: entries past the diagonal written"


def _eight_wave(B, H, S, D):
    """Whether prefill_attn_run takes the eight-wave kernel for int16 inputs of this shape."""
    return D == 128 and B * H * ((S + 255) // 256) >= 256


@pytest.mark.parametrize("offs", [None, [3]])
def test_int16_rotation_bit_exact_all_heads(offs):
    w = synth.WORKLOADS["i16_h32_s2048_d128"]
    announce("i16 rope", offs)
    q, k, v = synth.make_inputs(w)
    max_seq = w.seq_len + (offs[0] if offs else 0)
    attn = _i16_handle(w, max_seq)
    try:
        off_d = None if offs is None else torch.tensor(offs, dtype=torch.int32, device="cuda")
        for name, x in (("q", q), ("k", k)):
            xd = x.cuda()
            xr = torch.empty_like(xd)
            pa.prefill_attn_debug_rope_i16(attn.handle, w.batch, w.seq_len, xd, x.shape[2], off_d, xr)
            torch.cuda.synchronize()
            pos = np.arange(w.seq_len) + (offs[0] if offs else 0)
            want = oracle.rope_rotate_i16(x[0].numpy(), pos, w.rope_theta)
            assert np.array_equal(xr.cpu()[0].numpy().astype(np.int64), want), name
    finally:
        attn.close()


def test_int16_scores_bit_exact():
    """All 32 heads of the 1 x 32 x 2048 x 128 int16 workload, scores stored by
    the eight-wave two-group kernel that prefill_attn_run launches for it."""
    w = synth.WORKLOADS["i16_h32_s2048_d128"]
    assert _eight_wave(w.batch, w.n_heads, w.seq_len, w.head_dim)
    announce("i16 scores, eight-wave kernel")
    q, k, v = synth.make_inputs(w)
    attn = _i16_handle(w)
    try:
        qd, kd = to_dev(q, k)
        sc = _score_buffer(w.batch, w.n_heads, w.seq_len)
        pa.prefill_attn_debug_scores_i32(attn.handle, w.batch, w.seq_len, qd, kd, None, sc)
        assert attn.status() == pa.PA_OK
        pos = np.arange(w.seq_len)
        qr = oracle.rope_rotate_i16(q[0].numpy(), pos, w.rope_theta)
        kr = oracle.rope_rotate_i16(k[0].numpy(), pos, w.rope_theta)
        for h in range(w.n_heads):
            _assert_causal_scores(sc[0, h], oracle.scores_i32(qr[:, h], kr[:, h]), f"head {h}")
    finally:
        attn.close()


@pytest.mark.parametrize("D", [64, 128])
def test_int16_scores_ragged_gqa_offsets(D):
    """A small ragged GQA shape with offsets: the four-wave kernel's scores."""
    w = synth.Workload("i16_small", 2, 4, 2, 150, D, "i16", 1e4, 77, score_scale=2.0 ** -22 / 8)
    assert not _eight_wave(2, 4, 150, D)
    announce(w.name, D)
    q, k, v = synth.make_inputs(w)
    offs = [0, 40]
    attn = pa.PrefillAttention(4, 2, D, 190, 1e4)
    try:
        qd, kd = to_dev(q, k)
        od = torch.tensor(offs, dtype=torch.int32, device="cuda")
        sc = _score_buffer(2, 4, 150)
        pa.prefill_attn_debug_scores_i32(attn.handle, 2, 150, qd, kd, od, sc)
        assert attn.status() == pa.PA_OK
        for b in range(2):
            pos = np.arange(150) + offs[b]
            qr = oracle.rope_rotate_i16(q[b].numpy(), pos, 1e4)
            kr = oracle.rope_rotate_i16(k[b].numpy(), pos, 1e4)
            for h in range(4):
                _assert_causal_scores(sc[b, h], oracle.scores_i32(qr[:, h], kr[:, h // 2]), f"b{b} h{h}")
    finally:
        attn.close()


def test_int16_rotation_bit_exact_four_wave_staging():
    """The rope export at a shape whose prefill stages with 256 threads."""
    w = synth.Workload("i16_rope_small", 2, 3, 3, 203, 96, "i16", 1e4, 55)
    assert not _eight_wave(2, 3, 203, 96)
    announce(w.name)
    q, k, v = synth.make_inputs(w)
    offs = [0, 9]
    attn = pa.PrefillAttention(3, 3, 96, 212, 1e4)
    try:
        xd = k.cuda()
        xr = torch.empty_like(xd)
        od = torch.tensor(offs, dtype=torch.int32, device="cuda")
        pa.prefill_attn_debug_rope_i16(attn.handle, 2, 203, xd, 3, od, xr)
        assert attn.status() == pa.PA_OK
        for b in range(2):
            want = oracle.rope_rotate_i16(k[b].numpy(), np.arange(203) + offs[b], 1e4)
            assert np.array_equal(xr.cpu()[b].numpy().astype(np.int64), want), b
    finally:
        attn.close()


def test_int16_attention_output():
    """1 x 32 x 2048 x 128 int16: the whole O against the oracle."""
    w = synth.WORKLOADS["i16_h32_s2048_d128"]
    announce(w.name)
    q, k, v = synth.make_inputs(w)
    got = run_gpu(w, q, k, v).numpy()
    mx, mean = assert_close(got, oracle_full(w, q, k, v), "bf16")
    announce("margin", w.name, f"max {mx:.3e} mean {mean:.3e}")


# Plain head_dim 128 launches with at least 256 workgroups of 256 query rows
# run the int16 and in-kernel quantised variants on the eight-wave two-group
# kernel.
EIGHT_WAVE_INT = [
    # name, B, Hq, Hkv, S, D, dtype, offsets
    ("i16_8wave_d128_gqa_offsets", 2, 32, 8, 1100, 128, "i16", [0, 300]),
    ("i16_8wave_d128_paired", 1, 64, 16, 1800, 128, "i16", None),  # 8 blocks, the last of 8 rows: 256 pairs
    ("q16_8wave_d128_ragged", 1, 64, 8, 1030, 128, "bf16q", [7]),
    ("q16_8wave_d128_paired_odd", 1, 64, 8, 1700, 128, "bf16q", None),  # 7 blocks: the middle one alone
]


@pytest.mark.parametrize("case", EIGHT_WAVE_INT, ids=[c[0] for c in EIGHT_WAVE_INT])
def test_int_variants_eight_wave_full_compare(case):
    name, B, Hq, Hkv, S, D, dt, offs = case
    assert B * Hq * ((S + 255) // 256) >= 256
    announce(name)
    max_seq = S + (max(offs) if offs else 0)
    scale = 2.0 ** -22 / np.sqrt(D) if dt == "i16" else 0.0
    w = synth.Workload(name, B, Hq, Hkv, S, D, dt, 1e4, sum(map(ord, name)), score_scale=scale, max_seq=max_seq)
    q, k, v = synth.make_inputs(w)
    got = run_gpu(w, q, k, v, pos_offsets=offs)
    mx, mean = assert_close(got.numpy(), oracle_full(w, q, k, v, pos_offsets=offs), "bf16")
    announce(name, f"max {mx:.2e} mean {mean:.2e}")


def test_int16_degenerate_scale_small():
    """A large score scale makes the softmax nearly one-hot: exercises ties and argmax."""
    w = synth.Workload("i16_sharp", 1, 2, 2, 130, 128, "i16", 1e4, 88, score_scale=2.0 ** -8 / 11.3137085)
    announce(w.name)
    q, k, v = synth.make_inputs(w)
    got = run_gpu(w, q, k, v)
    want = oracle_full(w, q, k, v)
    assert_close(got.numpy(), want, "bf16")


# ------------------------------------------------------------ bf16 quantised in-kernel to int16

Q16_SCORE_CASES = [
    # name, B, Hq, Hkv, S, D, offsets
    ("q16_scores_d128_gqa", 2, 4, 2, 300, 128, [0, 21]),
    ("q16_scores_d96", 1, 2, 2, 200, 96, [5]),
    ("q16_scores_d64", 2, 2, 1, 130, 64, None),
]


@pytest.mark.parametrize("case", Q16_SCORE_CASES, ids=[c[0] for c in Q16_SCORE_CASES])
def test_quantised_scores_bit_exact(case):
    """The in-kernel codes (fp32 absmax, scale and round-half-even), their integer
    RoPE and the exact int32 scores, all bit-for-bit against the oracle."""
    name, B, Hq, Hkv, S, D, offs = case
    announce(name)
    w = synth.Workload(name, B, Hq, Hkv, S, D, "bf16q", 1e4, sum(map(ord, name)))
    q, k, v = synth.make_inputs(w)
    q[0, 3, 0] = 0  # an all-zero row quantises to zeros
    max_seq = S + (max(offs) if offs else 0)
    attn = pa.PrefillAttention(Hq, Hkv, D, max_seq, 1e4)
    try:
        qd, kd = to_dev(q, k)
        od = None if offs is None else torch.tensor(offs, dtype=torch.int32, device="cuda")
        sc = _score_buffer(B, Hq, S)
        pa.prefill_attn_debug_scores_q16(attn.handle, B, S, qd, kd, od, sc)
        assert attn.status() == pa.PA_OK
        qc, _ = oracle.quantize_rows_i16(q.float().numpy())
        kc, _ = oracle.quantize_rows_i16(k.float().numpy())
        for b in range(B):
            pos = np.arange(S) + (offs[b] if offs else 0)
            qr = oracle.rope_rotate_i16(qc[b], pos, 1e4)
            kr = oracle.rope_rotate_i16(kc[b], pos, 1e4)
            for h in range(Hq):
                _assert_causal_scores(sc[b, h], oracle.scores_i32(qr[:, h], kr[:, h // (Hq // Hkv)]), f"b{b} h{h}")
    finally:
        attn.close()


def test_quantised_scores_bit_exact_workload():
    """All 32 heads of the quantised 1 x 32 x 2048 x 128 workload, scores stored
    by the eight-wave kernel that PA_IN_BF16_Q16 runs at that shape."""
    w = synth.WORKLOADS["q16_bf16_h32_s2048_d128"]
    assert _eight_wave(w.batch, w.n_heads, w.seq_len, w.head_dim)
    announce(w.name, "scores")
    q, k, v = synth.make_inputs(w)
    attn = pa.PrefillAttention(w.n_heads, w.n_kv_heads, w.head_dim, w.seq_len, w.rope_theta)
    try:
        qd, kd = to_dev(q, k)
        sc = _score_buffer(1, w.n_heads, w.seq_len)
        pa.prefill_attn_debug_scores_q16(attn.handle, 1, w.seq_len, qd, kd, None, sc)
        assert attn.status() == pa.PA_OK
        qc, _ = oracle.quantize_rows_i16(q.float().numpy())
        kc, _ = oracle.quantize_rows_i16(k.float().numpy())
        pos = np.arange(w.seq_len)
        qr = oracle.rope_rotate_i16(qc[0], pos, w.rope_theta)
        kr = oracle.rope_rotate_i16(kc[0], pos, w.rope_theta)
        for h in range(w.n_heads):
            _assert_causal_scores(sc[0, h], oracle.scores_i32(qr[:, h], kr[:, h]), f"head {h}")
    finally:
        attn.close()


Q16_SMALL = [
    # name, B, Hq, Hkv, S, D, offsets
    ("q16_d128_ragged_gqa", 2, 4, 2, 333, 128, [0, 40]),
    ("q16_d96_ragged", 1, 4, 4, 257, 96, None),
    ("q16_d64_s1", 3, 2, 1, 1, 64, None),
]


@pytest.mark.parametrize("case", Q16_SMALL, ids=[c[0] for c in Q16_SMALL])
def test_quantised_attention_small_full_compare(case):
    name, B, Hq, Hkv, S, D, offs = case
    announce(name)
    max_seq = S + (max(offs) if offs else 0)
    w = synth.Workload(name, B, Hq, Hkv, S, D, "bf16q", 1e4, sum(map(ord, name)), max_seq=max_seq)
    q, k, v = synth.make_inputs(w)
    got = run_gpu(w, q, k, v, pos_offsets=offs)
    mx, mean = assert_close(got.numpy(), oracle_full(w, q, k, v, pos_offsets=offs), "bf16")
    announce(name, f"max {mx:.2e} mean {mean:.2e}")


def test_quantised_attention_workload():
    """1 x 32 x 2048 x 128 bf16 through the in-kernel quantisation: the whole O."""
    w = synth.WORKLOADS["q16_bf16_h32_s2048_d128"]
    announce(w.name)
    q, k, v = synth.make_inputs(w)
    got = run_gpu(w, q, k, v).numpy()
    mx, mean = assert_close(got, oracle_full(w, q, k, v), "bf16")
    announce("margin", w.name, f"max {mx:.3e} mean {mean:.3e}")


def test_quantised_cached_equals_quantised_prefill_bitwise():
    w = synth.Workload("q16_cached", 1, 4, 2, 300, 128, "bf16q", 1e4, 4321)
    announce(w.name)
    q, k, v = synth.make_inputs(w)
    attn = pa.PrefillAttention(4, 2, 128, 300, 1e4)
    try:
        qd, kd, vd = to_dev(q, k, v)
        o_plain = attn(qd, kd, vd, quantize=True)
        ident = torch.arange(300, dtype=torch.int32, device="cuda")[None, :]
        o_cached = attn.run_cached(qd, kd[0], vd[0], ident, quantize=True)
        torch.cuda.synchronize()
        assert attn.status() == pa.PA_OK
        assert torch.equal(o_plain, o_cached)
    finally:
        attn.close()


# ------------------------------------------------------------ int16 with the piecewise-linear softmax

PWL_SMALL = [
    # name, B, Hq, Hkv, S, D, offsets, score scale
    ("pwl_d128_gqa_ragged", 2, 4, 2, 300, 128, [0, 17], 2.0 ** -22 / 11.3137085),
    ("pwl_d96", 1, 2, 2, 257, 96, None, 2.0 ** -22 / 9.797959),
    ("pwl_d64_sharp", 1, 2, 1, 130, 64, None, 2.0 ** -16),  # logits spread far past the -8 cut-off
]


def _pwl_oracle(w, q, k, v, offs):
    return oracle.attention_i16_pwl(q.numpy(), k.numpy(), synth.to_f64(v), pos_offsets=offs,
                                    rope_theta=w.rope_theta, score_scale=w.score_scale)


def _pwl_gpu(w, q, k, v, offs=None, max_seq=None):
    attn = pa.PrefillAttention(w.n_heads, w.n_kv_heads, w.head_dim, max_seq or w.seq_len, w.rope_theta)
    try:
        qd, kd, vd = to_dev(q, k, v)
        od = None if offs is None else torch.tensor(offs, dtype=torch.int32, device="cuda")
        o = attn(qd, kd, vd, pos_offsets=od, score_scale=w.score_scale, pwl_softmax=True)
        torch.cuda.synchronize()
        assert attn.status() == pa.PA_OK
        return o.cpu().numpy()
    finally:
        attn.close()


@pytest.mark.parametrize("case", PWL_SMALL, ids=[c[0] for c in PWL_SMALL])
def test_pwl_softmax_small_full_compare(case):
    """Against the oracle's piecewise-linear softmax (same definition); the
    bar is the bf16 one, the weights being rounded to fp16 for P.V."""
    name, B, Hq, Hkv, S, D, offs, scale = case
    announce(name)
    max_seq = S + (max(offs) if offs else 0)
    w = synth.Workload(name, B, Hq, Hkv, S, D, "i16", 1e4, sum(map(ord, name)), score_scale=scale)
    q, k, v = synth.make_inputs(w)
    got = _pwl_gpu(w, q, k, v, offs, max_seq)
    mx, mean = assert_close(got, _pwl_oracle(w, q, k, v, offs), "bf16")
    announce(name, f"max {mx:.2e} mean {mean:.2e}")


def test_pwl_softmax_int16_workload():
    w = synth.WORKLOADS["i16_h32_s2048_d128"]
    announce(w.name, "pwl softmax")
    q, k, v = synth.make_inputs(w)
    got = _pwl_gpu(w, q, k, v)
    for h in (0, 13, 31):
        one = synth.workload(w.name, n_heads=1, n_kv_heads=1)
        want = _pwl_oracle(one, q[:, :, h:h + 1], k[:, :, h:h + 1], v[:, :, h:h + 1], None)
        assert_close(got[:, :, h:h + 1], want, "bf16")
