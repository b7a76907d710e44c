"""Runs on caller streams.  prefill_attn_run is asynchronous on the stream it is
given and a handle's tables are read-only after init, so runs may overlap on
several streams; they share only the handle's status word.  Each case runs the
same work interleaved on two streams (default priority) several times and
compares it bit for bit with the same runs made one after another on the
current stream.
"""

import pytest
import torch

import rope_causal_attention_amd as pa
import synth
from gpu_common import announce, need_gpu, to_dev

pytestmark = pytest.mark.gpu

REPEATS = 3


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _inputs(name, dtype, H, Hkv, S, D, seed):
    w = synth.Workload(name, 1, H, Hkv, S, D, dtype, 1e4, seed,
                       score_scale=2.0 ** -22 / D ** 0.5 if dtype == "i16" else 0.0)
    return w, to_dev(*synth.make_inputs(w))


def _on_streams(jobs):
    """jobs: (callable taking (out, stream), out tensor) pairs, one stream each,
    launched in turn REPEATS times with no synchronisation between them."""
    streams = [torch.cuda.Stream() for _ in jobs]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())  # the inputs were written on the current stream
    for _ in range(REPEATS):
        for (job, out), s in zip(jobs, streams):
            with torch.cuda.stream(s):
                job(out, s)
    torch.cuda.synchronize()


def test_one_handle_on_two_streams_bitwise():
    w, (q1, k1, v1) = _inputs("streams_a", "bf16", 8, 2, 1000, 96, 6001)
    _, (q2, k2, v2) = _inputs("streams_b", "bf16", 8, 2, 1000, 96, 6002)
    announce(w.name, "one handle, two streams")
    attn = pa.PrefillAttention(8, 2, 96, 1000, 1e4)
    try:
        ref1, ref2 = attn(q1, k1, v1), attn(q2, k2, v2)
        torch.cuda.synchronize()
        out1, out2 = torch.empty_like(ref1), torch.empty_like(ref2)
        _on_streams([(lambda o, s: attn(q1, k1, v1, out=o, stream=s), out1),
                     (lambda o, s: attn(q2, k2, v2, out=o, stream=s), out2)])
        assert attn.status() == pa.PA_OK
        assert torch.equal(out1, ref1) and torch.equal(out2, ref2)
    finally:
        attn.close()


def test_two_handles_of_different_types_on_two_streams_bitwise():
    wa, (qa, ka, va) = _inputs("streams_bf16_d128", "bf16", 16, 8, 700, 128, 6003)
    wb, (qb, kb, vb) = _inputs("streams_i16_d64", "i16", 4, 4, 900, 64, 6004)
    announce(wa.name, wb.name)
    ha = pa.PrefillAttention(16, 8, 128, 700, 1e4)
    hb = pa.PrefillAttention(4, 4, 64, 900, 1e4)
    try:
        ref_a = ha(qa, ka, va)
        ref_b = hb(qb, kb, vb, score_scale=wb.score_scale)
        torch.cuda.synchronize()
        out_a, out_b = torch.empty_like(ref_a), torch.empty_like(ref_b)
        _on_streams([(lambda o, s: ha(qa, ka, va, out=o, stream=s), out_a),
                     (lambda o, s: hb(qb, kb, vb, score_scale=wb.score_scale, out=o, stream=s), out_b)])
        assert ha.status() == pa.PA_OK and hb.status() == pa.PA_OK
        assert torch.equal(out_a, ref_a) and torch.equal(out_b, ref_b)
    finally:
        ha.close()
        hb.close()


def test_status_word_is_shared_between_streams():
    """A run whose positions leave the table, on one stream, beside a good run on
    another: the good run's O is unaffected, the bad one's is zero, and the
    handle's (shared) status word reports the range error."""
    w, (q, k, v) = _inputs("streams_status", "bf16", 4, 4, 256, 64, 6005)
    announce(w.name)
    attn = pa.PrefillAttention(4, 4, 64, 300, 1e4)
    try:
        ref = attn(q, k, v)
        torch.cuda.synchronize()
        bad_off = torch.tensor([100], dtype=torch.int32, device="cuda")  # 100 + 256 > 300
        out_good, out_bad = torch.empty_like(ref), torch.full_like(ref, 7.0)
        _on_streams([(lambda o, s: attn(q, k, v, out=o, stream=s), out_good),
                     (lambda o, s: attn(q, k, v, pos_offsets=bad_off, out=o, stream=s), out_bad)])
        assert attn.status() == pa.PA_ERANGE
        assert attn.status() == pa.PA_OK  # reading clears it
        assert torch.equal(out_good, ref)
        assert torch.all(out_bad == 0)
    finally:
        attn.close()
