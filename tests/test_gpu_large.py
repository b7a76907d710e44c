"""GPU parity at sizes beyond the named workloads.

  * 32K-token prompts (plus a ragged tail of 37) at head_dim 64, 96 and 128,
    with GQA, so the longest query rows run over 513 key tiles;
  * positions at the very end of the largest table init accepts (2^20 rows),
    for the bf16 and the int16 paths, and one past it;
  * launches of thousands of workgroups (a large batch of GQA heads packed four
    to a workgroup, and a large MHA batch);
  * decode over a 65,536-token context, and a cached prefill chunk after a
    60,000-token prefix (the fused cache update, split-K chosen by the library).

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
from gpu_common import announce, assert_close, errors, need_gpu, oracle_full, oracle_rows, run_gpu, sample_rows, to_dev

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


def test_decode_long_context():
    """Two sequences with 65,536 and 40,001 cached tokens, 32 query / 8 KV heads,
    head_dim 128, a bf16 paged cache of shuffled 64-slot blocks; the library
    picks the split.  Decode computes in fp32: the fp32 bar, 1e-5."""
    from test_gpu_decode import TOL, Decode
    c = Decode("dec_ctx65536", 2, 32, 8, 128, "bf16", [65535, 40000], block=64)
    announce(c.name)
    mx, mean = errors(c.run().numpy(), c.oracle())
    announce("margin", c.name, f"max {mx:.3e} mean {mean:.3e}")
    assert mx <= TOL, mx


def test_cached_prefill_after_a_long_prefix():
    """A 1000-token chunk after 60,000 cached tokens (GQA 8/2, head_dim 96, bf16,
    shuffled 64-slot blocks) through prefill_attn_run_cached_update with the
    split chosen by the library: the chunk's rows land in their slots bit for
    bit, and sampled output rows match the oracle."""
    B, Hq, Hkv, D, block, P, S = 1, 8, 2, 96, 64, 60000, 1000
    T = P + S
    need = (T + block - 1) // block
    n_slots = (need + 3) * block
    rng = np.random.default_rng(5300)
    kv_map = oracle.paged_index_map(rng.permutation(need + 3)[:need], block, T)[None].astype(np.int32)
    g = torch.Generator().manual_seed(5300)
    kc = torch.randn((n_slots, Hkv, D), generator=g).to(torch.bfloat16)
    vc = torch.randn((n_slots, Hkv, D), generator=g).to(torch.bfloat16)
    q = torch.randn((B, S, Hq, D), generator=g).to(torch.bfloat16)
    kn = torch.randn((B, S, Hkv, D), generator=g).to(torch.bfloat16)
    vn = torch.randn((B, S, Hkv, D), generator=g).to(torch.bfloat16)
    announce("cached_prefix60000_chunk1000_d96")
    attn = pa.PrefillAttention(Hq, Hkv, D, T, 1e4)
    try:
        kcd, vcd = kc.cuda(), vc.cuda()
        ws = torch.empty(pa.prefill_attn_run_cached_workspace_size(attn.handle, B, S, 16), dtype=torch.uint8,
                         device="cuda")
        off = torch.tensor([P], dtype=torch.int32, device="cuda")
        o = attn.run_cached_update(q.cuda(), kn.cuda(), vn.cuda(), kcd, vcd, torch.from_numpy(kv_map).cuda(),
                                   pos_offsets=off, n_split=0, workspace=ws)
        torch.cuda.synchronize()
        assert attn.status() == pa.PA_OK
        o, kcd, vcd = o.cpu(), kcd.cpu(), vcd.cpu()
    finally:
        attn.close()
    bits = lambda t: t.view(torch.int16).numpy()  # noqa: E731
    k_want, v_want = oracle.kv_cache_update(bits(kc), bits(vc), bits(kn), bits(vn), kv_map, prefix=[P])
    assert np.array_equal(bits(kcd), k_want) and np.array_equal(bits(vcd), v_want)
    rows = {(0, h, i) for h in (0, 3, 7) for i in (0, 1, 63, 64, 500, S - 1)}
    rows |= {(0, int(rng.integers(Hq)), int(rng.integers(S))) for _ in range(12)}
    rows = sorted(rows)
    f = synth.to_f64
    want = oracle.attention_cached_rows(f(q), f(kcd), f(vcd), kv_map, rows, prefix=[P])
    mx, mean = assert_close(_rows_of(o, rows), want, "bf16")
    announce("margin", "cached_prefix60000_chunk1000_d96", f"max {mx:.3e} mean {mean:.3e} over {len(rows)} rows")
