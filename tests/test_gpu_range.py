"""GPU tests of the documented value ranges (include/prefill_attn.h, the input
types): what the kernels do when an input leaves the range they compute in.

  * PA_IN_BF16 rounds Q' (scaled), K' = RoPE(K) and V to fp16 for the matrix
    cores.  A K' beyond 65504, or any O that comes out non-finite (an fp16 V or
    Q' that overflowed), sets the status word: prefill_attn_status returns
    PA_EOVERFLOW.  Values inside the range leave it clear.
  * PA_IN_I16 splits each rotated Q'/K' value into int8 digits, exact for
    values in [-16448, 16319].  A value outside sets PA_EOVERFLOW; the edge values
    themselves are exact (scores bit-equal to the oracle).
"""

import numpy as np
import pytest
import torch

import oracle
import rope_causal_attention_amd as pa
import synth
from gpu_common import announce, assert_close, need_gpu, oracle_full, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _run(w, q, k, v, score_scale=0.0):
    """O (CPU) and the status code of one prefill_attn_run."""
    attn = pa.PrefillAttention(w.n_heads, w.n_kv_heads, w.head_dim, w.seq_len, w.rope_theta)
    try:
        qd, kd, vd = to_dev(q, k, v)
        o = attn(qd, kd, vd, score_scale=score_scale)
        return o.cpu(), attn.status()
    finally:
        attn.close()


# name, B, Hq, Hkv, S, D: a four-wave shape and an eight-wave one
BF16_SHAPES = [("bf16_range_4wave", 1, 2, 2, 100, 64), ("bf16_range_8wave", 1, 64, 64, 1024, 64)]


@pytest.mark.parametrize("shape", BF16_SHAPES, ids=[s[0] for s in BF16_SHAPES])
@pytest.mark.parametrize("where", ["k", "v", "q"])
def test_bf16_overflow_sets_status(shape, where):
    name, B, H, Hkv, S, D = shape
    w = synth.Workload(name, B, H, Hkv, S, D, "bf16", 1e4, 31)
    q, k, v = synth.make_inputs(w)
    big = 3.0e5  # fp16 overflows at 65520; bf16 holds it
    if where == "k":
        k[0, 50, 1, 0:2] = big  # a rotated pair of norm big * sqrt 2: one half is at least big
    elif where == "v":
        v[0, 30, 1, 5] = big
    else:
        q[0, 70, 1, 0:2] = big
    announce(name, where)
    o, st = _run(w, q, k, v, score_scale=1.0 if where == "q" else 0.0)
    assert st == pa.PA_EOVERFLOW, (where, st)
    # heads other than head 1 never see the value: untouched and finite
    assert torch.isfinite(o[:, :, 0]).all()


def test_bf16_largest_values_inside_the_range():
    """bf16 65280 (the largest bf16 value below the fp16 limit) in V, and K
    pairs whose rotation stays below 65504: status clear, O finite and equal
    to the oracle within the bf16 tolerance scaled by the value size."""
    w = synth.Workload("bf16_range_edge", 1, 2, 2, 100, 64, "bf16", 1e4, 32)
    q, k, v = synth.make_inputs(w)
    v[0, 30, 1, 5] = 65280.0
    k[0, 50, 1, 0] = 46080.0  # |rotated| <= 46080 sqrt 2 = 65167
    k[0, 50, 1, 1] = 0.0
    announce(w.name)
    o, st = _run(w, q, k, v)
    assert st == pa.PA_OK
    assert torch.isfinite(o).all()
    want = oracle_full(w, q, k, v)
    err = np.abs(o.numpy().astype(np.float64) - want)
    assert err.max() <= 1e-2 * 65280 / 4, err.max()


def _i16_case(x0, where="q"):
    w = synth.Workload("i16_digit_edge", 1, 2, 2, 70, 64, "i16", 1e4, 33, score_scale=2.0 ** -22 / 8)
    q, k, v = synth.make_inputs(w)
    t = q if where == "q" else k
    t[0, 0, 1, 0] = x0  # position 0: C = 2^14, S = 0, so the rotated value is x0 itself
    t[0, 0, 1, 1] = 0
    return w, q, k, v


@pytest.mark.parametrize("x0", [16319, -16448])
@pytest.mark.parametrize("where", ["q", "k"])
def test_int16_digit_range_edges_exact(x0, where):
    w, q, k, v = _i16_case(x0, where)
    announce(w.name, where, x0)
    attn = pa.PrefillAttention(2, 2, 64, 70, 1e4)
    try:
        qd, kd, vd = to_dev(q, k, v)
        o = attn(qd, kd, vd, score_scale=w.score_scale)
        assert attn.status() == pa.PA_OK
        sc = torch.full((1, 2, 70, 70), -2 ** 31, dtype=torch.int32, device="cuda")
        pa.prefill_attn_debug_scores_i32(attn.handle, 1, 70, qd, kd, None, sc)
        assert attn.status() == pa.PA_OK
    finally:
        attn.close()
    pos = np.arange(70)
    qr = oracle.rope_rotate_i16(q[0].numpy(), pos, 1e4)
    kr = oracle.rope_rotate_i16(k[0].numpy(), pos, 1e4)
    assert (qr if where == "q" else kr)[0, 1, 0] == x0
    want = oracle.scores_i32(qr[:, 1], kr[:, 1])
    got = sc[0, 1].cpu().numpy().astype(np.int64)
    low = np.tril(np.ones((70, 70), dtype=bool))
    assert np.array_equal(got[low], want[low])
    assert_close(o.cpu().numpy(), oracle_full(w, q, k, v), "bf16")


@pytest.mark.parametrize("x0", [16320, -16449, 20000])
@pytest.mark.parametrize("where", ["q", "k"])
def test_int16_digit_range_exceeded_sets_status(x0, where):
    w, q, k, v = _i16_case(x0, where)
    announce(w.name, where, x0)
    o, st = _run(w, q, k, v, score_scale=w.score_scale)
    assert st == pa.PA_EOVERFLOW, st
    attn = pa.PrefillAttention(2, 2, 64, 70, 1e4)
    try:
        x = (q if where == "q" else k).cuda()
        xr = torch.empty_like(x)
        pa.prefill_attn_debug_rope_i16(attn.handle, 1, 70, x, 2, None, xr)
        assert attn.status() == pa.PA_EOVERFLOW
    finally:
        attn.close()
