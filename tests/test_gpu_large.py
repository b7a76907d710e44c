"""GPU parity at sizes beyond the named workloads.

  * 32K-token prompts (plus a ragged tail of 37) at head_dim 64, 96 and 128,
    with GQA, so the longest query rows run over 513 key tiles;
  * positions at the very end of the largest table init accepts (2^20 rows),
    for the bf16 and the int16 paths, and one past it;
  * launches of thousands of workgroups (a large batch of GQA heads packed four
    to a workgroup, and a large MHA batch).

The oracle evaluates sampled output rows one by one (oracle.attention_rows and
its int16 twin), always including the first and last rows, rows at the tile
and block boundaries, and the ragged tail.
"""

import numpy as np
import pytest
import torch

import oracle
import rope_causal_attention_amd as pa
import synth
from gpu_common import announce, assert_close, need_gpu, oracle_full, oracle_rows, run_gpu, sample_rows, to_dev

pytestmark = pytest.mark.gpu

MAX_SEQ = 1 << 20  # the largest max_seq prefill_attn_init accepts


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _rows_of(got, rows):
    return np.stack([got[b, i, h].numpy() for b, h, i in rows])


LONG = [("long_s32805_d64", 64), ("long_s32805_d96", 96), ("long_s32805_d128", 128)]


@pytest.mark.parametrize("name,D", LONG, ids=[n for n, _ in LONG])
def test_long_sequence_sampled_rows(name, D):
    S = 32768 + 37  # a multiple of neither 64 nor 256
    w = synth.Workload(name, 1, 4, 2, S, D, "bf16", 1e4, 5000 + D)
    announce(name)
    q, k, v = synth.make_inputs(w)
    got = run_gpu(w, q, k, v)
    rows = set(sample_rows(w, 16, seed=D))
    rows |= {(0, h, i) for h in (0, 3) for i in (63, 64, 255, 256, 32767, 32768, S - 1)}
    rows = sorted(rows)
    mx, mean = assert_close(_rows_of(got, rows), oracle_rows(w, q, k, v, rows), "bf16")
    announce("margin", name, f"max {mx:.3e} mean {mean:.3e} over {len(rows)} rows")


@pytest.mark.parametrize("dtype", ["bf16", "i16"])
def test_positions_at_the_end_of_the_largest_table(dtype):
    """Batch element 0 ends exactly at the last table row, element 1 starts at 0;
    one more position is out of range (status set, that element's O zero)."""
    S, D = 300, 64
    w = synth.Workload(f"table_end_{dtype}", 2, 2, 2, S, D, dtype, 1e4, 5100,
                       score_scale=2.0 ** -22 / 8 if dtype == "i16" else 0.0)
    announce(w.name, MAX_SEQ)
    q, k, v = synth.make_inputs(w)
    offs = [MAX_SEQ - S, 0]
    attn = pa.PrefillAttention(2, 2, D, MAX_SEQ, 1e4)
    try:
        qd, kd, vd = to_dev(q, k, v)
        got = run_gpu(w, q, k, v, pos_offsets=offs, attn=attn)
        assert_close(got.numpy(), oracle_full(w, q, k, v, pos_offsets=np.array(offs)), dtype)
        if dtype == "i16":
            sc = torch.full((2, 2, S, S), -2 ** 31, dtype=torch.int32, device="cuda")
            off_d = torch.tensor(offs, dtype=torch.int32, device="cuda")
            pa.prefill_attn_debug_scores_i32(attn.handle, 2, S, qd, kd, off_d, sc)
            assert attn.status() == pa.PA_OK
            low = np.tril(np.ones((S, S), dtype=bool))
            for b in range(2):
                pos = offs[b] + np.arange(S)
                qr = oracle.rope_rotate_i16(q[b].numpy(), pos, 1e4)
                kr = oracle.rope_rotate_i16(k[b].numpy(), pos, 1e4)
                for h in range(2):
                    want = oracle.scores_i32(qr[:, h], kr[:, h])
                    assert np.array_equal(sc[b, h].cpu().numpy().astype(np.int64)[low], want[low]), (b, h)
        # one position past the table: element 0 is zeroed and the status set
        off_bad = torch.tensor([MAX_SEQ - S + 1, 0], dtype=torch.int32, device="cuda")
        o = attn(qd, kd, vd, pos_offsets=off_bad, score_scale=w.score_scale)
        assert attn.status() == pa.PA_ERANGE
        o = o.cpu()
        assert torch.all(o[0] == 0)
        assert_close(o[1:].numpy(), oracle_full(w, q[1:], k[1:], v[1:]), dtype)
    finally:
        attn.close()


# name, B, Hq, Hkv, S, D: GQA heads packed four to a workgroup (2112 workgroups),
# and a large MHA batch on the paired two-group kernel (768 workgroups of two blocks)
MANY = [("many_gqa_b48_h16kv4_s700_d96", 48, 16, 4, 700, 96), ("many_mha_b96_h8_s300_d128", 96, 8, 8, 300, 128)]


@pytest.mark.parametrize("case", MANY, ids=[c[0] for c in MANY])
def test_many_workgroups_sampled_rows(case):
    name, B, Hq, Hkv, S, D = case
    w = synth.Workload(name, B, Hq, Hkv, S, D, "bf16", 1e6, 5200 + D)
    announce(name)
    q, k, v = synth.make_inputs(w)
    got = run_gpu(w, q, k, v)
    rows = set(sample_rows(w, 40, seed=B))
    rows |= {(B - 1, h, i) for h in (0, Hq - 1) for i in (0, 63, 64, 255, 256, S - 1)}
    rows = sorted(rows)
    mx, mean = assert_close(_rows_of(got, rows), oracle_rows(w, q, k, v, rows), "bf16")
    announce("margin", name, f"max {mx:.3e} mean {mean:.3e} over {len(rows)} rows")
