"""GPU property tests: exact invariants of the fused kernel, edge cases and
error paths through the C-ABI (no oracle needed for most of them)."""

import ctypes

import numpy as np
import pytest
import torch

import rope_causal_attention_amd as pa
import synth
from gpu_common import announce, assert_close, need_gpu, oracle_full, run_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _w(dt, B=2, Hq=4, Hkv=2, S=200, D=128, theta=1e4, seed=5):
    return synth.Workload(f"prop_{dt}", B, Hq, Hkv, S, D, dt, theta, seed,
                          score_scale=(2.0 ** -22 / np.sqrt(D)) if dt == "i16" else 0.0)


@pytest.mark.parametrize("dt", ["f32", "bf16", "i16"])
def test_first_row_is_first_value_row_bitwise(dt):
    announce("row0", dt)
    w = _w(dt)
    q, k, v = synth.make_inputs(w)
    o = run_gpu(w, q, k, v)
    g = w.n_heads // w.n_kv_heads
    for h in range(w.n_heads):
        assert torch.equal(o[:, 0, h], v[:, 0, h // g].float())


# V = I (S <= D): O is the probability matrix itself.  Four-wave and eight-wave shapes.
IDENTITY_SHAPES = [("4wave", 1, 4, 2), ("8wave", 2, 128, 128)]


@pytest.mark.parametrize("shape", IDENTITY_SHAPES, ids=[s[0] for s in IDENTITY_SHAPES])
@pytest.mark.parametrize("dt", ["f32", "bf16", "i16"])
def test_identity_values_give_the_probabilities(dt, shape):
    """V = I makes O[i, j] = P[i, j]: entries past the diagonal exactly 0
    (masked keys weigh exactly nothing), rows summing to 1, and the
    probabilities equal to the oracle's (the oracle with V = I)."""
    name, B, Hq, Hkv = shape
    S, D = 96, 128
    announce("v=I", dt, name)
    w = _w(dt, B=B, Hq=Hq, Hkv=Hkv, S=S, D=D)
    q, k, v = synth.make_inputs(w)
    eye = torch.zeros(S, D)
    eye[:, :S] = torch.eye(S)
    v = eye[None, :, None, :].expand(B, S, Hkv, D).contiguous().to(v.dtype)
    o = run_gpu(w, q, k, v)
    p = o[..., :S].double()  # [B][S][Hq][S]
    upper = torch.triu(torch.ones(S, S, dtype=torch.bool), diagonal=1)
    assert torch.all(p.permute(0, 2, 1, 3)[:, :, upper] == 0)
    assert torch.all(o[..., S:] == 0)
    assert float((p.sum(-1) - 1).abs().max()) <= 1e-5
    assert_close(o.numpy(), oracle_full(w, q, k, v), "f32" if dt == "f32" else "bf16")


@pytest.mark.parametrize("dt", ["f32", "bf16", "i16"])
def test_constant_values_give_constant_output(dt):
    announce("v=1", dt)
    w = _w(dt, S=300)
    q, k, v = synth.make_inputs(w)
    v = torch.ones_like(v)
    o = run_gpu(w, q, k, v)
    assert float((o - 1).abs().max()) <= 1e-6


@pytest.mark.parametrize("dt", ["f32", "bf16", "i16"])
def test_gqa_equals_mha_with_repeated_kv_bitwise(dt):
    announce("gqa", dt)
    w = _w(dt, Hq=6, Hkv=2, S=170, D=96)
    q, k, v = synth.make_inputs(w)
    o = run_gpu(w, q, k, v)
    w2 = synth.Workload(w.name, w.batch, 6, 6, w.seq_len, 96, dt, w.rope_theta, w.seed, score_scale=w.score_scale)
    o2 = run_gpu(w2, q, k.repeat_interleave(3, dim=2).contiguous(), v.repeat_interleave(3, dim=2).contiguous())
    assert torch.equal(o, o2)


@pytest.mark.parametrize("dt", ["bf16", "i16"])
def test_batch_elements_are_independent_bitwise(dt):
    announce("batch", dt)
    w = _w(dt, B=3, S=250, D=64)
    q, k, v = synth.make_inputs(w)
    offs = [0, 9, 2]
    o = run_gpu(w, q, k, v, pos_offsets=offs, max_seq=260)
    for b in range(3):
        w1 = synth.Workload(w.name, 1, w.n_heads, w.n_kv_heads, w.seq_len, 64, dt, w.rope_theta, w.seed,
                            score_scale=w.score_scale)
        o1 = run_gpu(w1, q[b:b + 1].contiguous(), k[b:b + 1].contiguous(), v[b:b + 1].contiguous(),
                     pos_offsets=[offs[b]], max_seq=260)
        assert torch.equal(o[b:b + 1], o1)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_offsets_match_oracle_and_barely_move_output(dt):
    announce("offsets", dt)
    w = _w(dt, B=2, S=180, D=64)
    q, k, v = synth.make_inputs(w)
    max_seq = 4096
    offs = [max_seq - 180, 1234]
    o_off = run_gpu(w, q, k, v, pos_offsets=offs, max_seq=max_seq)
    assert_close(o_off.numpy(), oracle_full(w, q, k, v, pos_offsets=offs), dt)
    o0 = run_gpu(w, q, k, v, max_seq=max_seq)
    assert_close(o_off.numpy(), o0.numpy(), dt)


def test_out_of_range_offsets_zero_the_element_and_report():
    announce("erange")
    w = _w("bf16", B=2, S=64, D=64)
    q, k, v = synth.make_inputs(w)
    attn = pa.PrefillAttention(w.n_heads, w.n_kv_heads, 64, 100, 1e4)
    try:
        qd, kd, vd = to_dev(q, k, v)
        out = torch.full(q.shape, 7.0, dtype=torch.float32, device="cuda")
        off = torch.tensor([36, 37], dtype=torch.int32, device="cuda")  # 37 + 64 > 100
        attn(qd, kd, vd, pos_offsets=off, out=out)
        assert attn.status() == pa.PA_ERANGE
        assert attn.status() == pa.PA_OK  # cleared
        o = out.cpu()
        assert torch.all(o[1] == 0)
        assert torch.all(torch.isfinite(o[0])) and not torch.all(o[0] == 0)
        off = torch.tensor([-1, 0], dtype=torch.int32, device="cuda")
        attn(qd, kd, vd, pos_offsets=off, out=out)
        assert attn.status() == pa.PA_ERANGE
        assert torch.all(out.cpu()[0] == 0)
    finally:
        attn.close()


# Eight-wave launches: plain order, paired blocks, and GQA head packing
# (two query heads of a KV head per workgroup), paired and not.
EIGHT_WAVE = [
    # name, Hq, Hkv
    ("pack_unpaired", 32, 16),
    ("pack_paired", 64, 32),
    ("mha_paired", 64, 64),
]


@pytest.mark.parametrize("name,Hq,Hkv", EIGHT_WAVE, ids=[c[0] for c in EIGHT_WAVE])
def test_out_of_range_offsets_eight_wave(name, Hq, Hkv):
    """Element 1's positions leave the table: every head of it is zero, the
    status is reported, and element 0 equals its own single-element run."""
    announce("erange8", name)
    B, S, D, max_seq = 2, 1024, 64, 1100
    assert B * Hq * (S // 256) >= 256
    w = synth.Workload(name, B, Hq, Hkv, S, D, "bf16", 1e4, sum(map(ord, name)), max_seq=max_seq)
    q, k, v = synth.make_inputs(w)
    attn = pa.PrefillAttention(Hq, Hkv, D, max_seq, 1e4)
    try:
        qd, kd, vd = to_dev(q, k, v)
        out = torch.full(q.shape, 7.0, dtype=torch.float32, device="cuda")
        off = torch.tensor([50, 77], dtype=torch.int32, device="cuda")  # 77 + 1024 > 1100
        attn(qd, kd, vd, pos_offsets=off, out=out)
        assert attn.status() == pa.PA_ERANGE
        o = out.cpu()
        assert torch.all(o[1] == 0)
        o0 = attn(qd[:1].contiguous(), kd[:1].contiguous(), vd[:1].contiguous(),
                  pos_offsets=torch.tensor([50], dtype=torch.int32, device="cuda")).cpu()
        assert attn.status() == pa.PA_OK
        assert torch.equal(o[:1], o0)
    finally:
        attn.close()


def test_gqa_head_packing_equals_mha_with_repeated_kv_bitwise():
    """Two query heads per KV head on the eight-wave kernel (packed) against
    the same attention with K/V repeated per query head (unpacked)."""
    announce("gqa8")
    w = synth.Workload("gqa8", 1, 32, 16, 2048, 64, "bf16", 1e4, 4242)
    q, k, v = synth.make_inputs(w)
    o = run_gpu(w, q, k, v)
    w2 = synth.Workload("gqa8", 1, 32, 32, 2048, 64, "bf16", 1e4, 4242)
    o2 = run_gpu(w2, q, k.repeat_interleave(2, dim=2).contiguous(), v.repeat_interleave(2, dim=2).contiguous())
    assert torch.equal(o, o2)


def test_empty_inputs_are_noops():
    attn = pa.PrefillAttention(2, 2, 64, 16, 1e4)
    try:
        pa.prefill_attn_run(attn.handle, pa.PA_IN_BF16, 0, 16, None, None, None, None, None)
        pa.prefill_attn_run(attn.handle, pa.PA_IN_BF16, 3, 0, None, None, None, None, None)
        assert attn.status() == pa.PA_OK
    finally:
        attn.close()


def test_max_seq_boundary():
    announce("max_seq")
    w = _w("bf16", B=1, Hq=2, Hkv=2, S=257, D=96)
    q, k, v = synth.make_inputs(w)
    o = run_gpu(w, q, k, v, max_seq=257)
    assert_close(o.numpy(), oracle_full(w, q, k, v), "bf16")
    attn = pa.PrefillAttention(2, 2, 96, 257, 1e4)
    try:
        qd, kd, vd = to_dev(q, k, v)
        out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        off = torch.tensor([1], dtype=torch.int32, device="cuda")
        attn(qd, kd, vd, pos_offsets=off, out=out)
        assert attn.status() == pa.PA_ERANGE
    finally:
        attn.close()


def test_invalid_arguments_return_status_codes():
    lib = pa.load_library()
    attn = pa.PrefillAttention(4, 2, 128, 64, 1e4)
    try:
        buf = torch.zeros(1 << 16, dtype=torch.float32, device="cuda")
        p = buf.data_ptr()
        h = attn.handle
        s = torch.cuda.current_stream().cuda_stream
        run = lambda *a: lib.prefill_attn_run(h, *a)  # noqa: E731
        assert run(pa.PA_IN_BF16, 1, 65, p, p, p, None, p, 0.0, s) == pa.PA_EINVAL      # seq > max_seq
        assert run(pa.PA_IN_BF16, -1, 8, p, p, p, None, p, 0.0, s) == pa.PA_EINVAL      # negative batch
        assert run(7, 1, 8, p, p, p, None, p, 0.0, s) == pa.PA_EINVAL                   # unknown dtype
        assert run(pa.PA_IN_BF16, 1, 8, p + 2, p, p, None, p, 0.0, s) == pa.PA_EINVAL   # misaligned q
        assert run(pa.PA_IN_BF16, 1, 8, p, p, p, p + 2, p, 0.0, s) == pa.PA_EINVAL      # misaligned offsets
        assert run(pa.PA_IN_BF16, 1, 8, p, None, p, None, p, 0.0, s) == pa.PA_EINVAL    # null k
        assert run(pa.PA_IN_BF16, 1, 8, p, p, p, None, p, float("nan"), s) == pa.PA_EINVAL
        assert lib.prefill_attn_debug_rope_i16(h, 1, 8, p, 0, None, p, s) == pa.PA_EINVAL
        torch.cuda.synchronize()
        assert attn.status() == pa.PA_OK
    finally:
        attn.close()


@pytest.mark.parametrize("dt", ["bf16", "i16", "f32"])
def test_repeated_runs_are_bitwise_identical(dt):
    w = _w(dt, B=1, Hq=8, Hkv=8, S=700, D=128 if dt != "f32" else 64)
    q, k, v = synth.make_inputs(w)
    attn = pa.PrefillAttention(w.n_heads, w.n_kv_heads, w.head_dim, w.seq_len, w.rope_theta)
    try:
        qd, kd, vd = to_dev(q, k, v)
        a = attn(qd, kd, vd, score_scale=w.score_scale)
        b = attn(qd, kd, vd, score_scale=w.score_scale)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
    finally:
        attn.close()
