"""Shared helpers for the GPU tests: device inputs, oracle comparisons."""

import sys

import numpy as np
import pytest
import torch

import oracle
import rope_causal_attention_amd as pa
import synth

# Tolerances: fp32 inputs max-abs 1e-5; bf16 (and the int16 variant's output)
# max-abs 1e-2 and mean-abs 1e-3, over every element of O.
TOL_F32_MAX = 1e-5
TOL_BF16_MAX = 1e-2
TOL_BF16_MEAN = 1e-3


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this process")


def announce(*parts):
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


def to_dev(*ts):
    return [t.cuda() for t in ts]


def errors(got, want):
    d = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64))
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def assert_close(got, want, dtype):
    mx, mean = errors(got, want)
    if dtype == "f32":
        assert mx <= TOL_F32_MAX, f"max-abs {mx:.3e} > {TOL_F32_MAX}"
    else:
        assert mx <= TOL_BF16_MAX and mean <= TOL_BF16_MEAN, f"max-abs {mx:.3e}, mean-abs {mean:.3e}"
    return mx, mean


def run_gpu(w, q, k, v, pos_offsets=None, score_scale=None, attn=None, max_seq=None):
    """Run the library on CPU tensors (copied to the device); returns O on the CPU."""
    own = attn is None
    if own:
        attn = pa.PrefillAttention(w.n_heads, w.n_kv_heads, w.head_dim, max_seq or w.max_seq or w.seq_len,
                                   w.rope_theta)
    try:
        qd, kd, vd = to_dev(q, k, v)
        off = None if pos_offsets is None else torch.tensor(pos_offsets, dtype=torch.int32, device="cuda")
        o = attn(qd, kd, vd, pos_offsets=off, score_scale=w.score_scale if score_scale is None else score_scale,
                 quantize=w.dtype == "bf16q")
        torch.cuda.synchronize()
        assert attn.status() == pa.PA_OK
        return o.cpu()
    finally:
        if own:
            attn.close()


def oracle_full(w, q, k, v, pos_offsets=None):
    if w.dtype == "bf16q":
        return oracle.attention_i16_quantized(q.float().numpy(), k.float().numpy(), synth.to_f64(v),
                                              pos_offsets=pos_offsets, rope_theta=w.rope_theta,
                                              score_scale=w.score_scale or None)
    if w.dtype == "i16":
        return oracle.attention_i16(synth.to_f64(q), synth.to_f64(k), synth.to_f64(v), pos_offsets=pos_offsets,
                                    rope_theta=w.rope_theta, score_scale=w.score_scale)
    scale = w.score_scale or None
    return oracle.attention(synth.to_f64(q), synth.to_f64(k), synth.to_f64(v), pos_offsets=pos_offsets,
                            rope_theta=w.rope_theta, scale=scale)


def oracle_rows(w, q, k, v, rows, pos_offsets=None):
    if w.dtype == "bf16q":
        return oracle.attention_i16_quantized_rows(q.float().numpy(), k.float().numpy(), v.float().numpy(), rows,
                                                   pos_offsets=pos_offsets, rope_theta=w.rope_theta,
                                                   score_scale=w.score_scale or None)
    if w.dtype == "i16":
        return oracle.attention_i16_rows(q.numpy(), k.numpy(), synth.to_f64(v), rows, pos_offsets=pos_offsets,
                                         rope_theta=w.rope_theta, score_scale=w.score_scale)
    return oracle.attention_rows(q.float().numpy(), k.float().numpy(), v.float().numpy(), rows,
                                 pos_offsets=pos_offsets, rope_theta=w.rope_theta, scale=w.score_scale or None)


def sample_rows(w, n, seed):
    """Rows (b, h, i) spread over the whole output, always including the extremes."""
    rng = np.random.default_rng(seed)
    rows = {(0, 0, 0), (w.batch - 1, w.n_heads - 1, w.seq_len - 1), (0, w.n_heads - 1, w.seq_len - 1),
            (w.batch - 1, 0, w.seq_len // 2)}
    while len(rows) < n:
        rows.add((int(rng.integers(w.batch)), int(rng.integers(w.n_heads)), int(rng.integers(w.seq_len))))
    return sorted(rows)
