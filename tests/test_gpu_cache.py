"""GPU parity of the KV-cache path: kv_cache_update and cached (chunked)
prefill through the C-ABI, against the fp64 oracle and against the plain
prefill path.

* the cache update is byte work: compared bit for bit;
* a cached run with the identity map and no prefix is the plain prefill and
  must match it bit for bit (same kernels, only the key addressing differs);
* chunked prefill through ring and paged maps, with ragged prefixes and
  garbage in unused slots, is compared with the oracle at the tolerances of
  the plain path (fp32 max-abs 1e-5; bf16 and int16 output max-abs 1e-2,
  mean-abs 1e-3), and with the plain prefill of the whole sequence.
"""

import numpy as np
import pytest
import torch

import oracle
import rope_causal_attention_amd as pa
import synth
from gpu_common import announce, assert_close, errors, need_gpu

pytestmark = pytest.mark.gpu

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "i16": torch.int16}


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _seed(name):
    return sum(map(ord, name))


def _score_scale(dt, D):
    return 2.0 ** -22 / np.sqrt(D) if dt == "i16" else 0.0


def _garbage(shape, dt, seed):
    g = torch.Generator().manual_seed(seed)
    if dt == "i16":
        return torch.randint(-2048, 2048, shape, generator=g, dtype=torch.int16)
    return (torch.randn(shape, generator=g) * 4.0).to(TORCH_DT[dt])


def _maps(layout, B, width, n_slots, seed, block=16):
    """Distinct slots for every (b, logical position < width)."""
    rng = np.random.default_rng(seed)
    if layout == "identity":
        assert B == 1
        return np.arange(width, dtype=np.int32)[None, :]
    if layout == "ring":
        per = n_slots // B
        return np.stack([oracle.ring_index_map(per, int(rng.integers(per)), width) + b * per
                         for b in range(B)]).astype(np.int32)
    assert layout == "paged"
    nb = n_slots // block
    blocks = rng.permutation(nb)
    need = (width + block - 1) // block
    return np.stack([oracle.paged_index_map(blocks[b * need:(b + 1) * need], block, width)
                     for b in range(B)]).astype(np.int32)


class Case:
    """Full logical sequences, a cache holding them, and the chunk's queries."""

    def __init__(self, name, B, Hq, Hkv, D, dt, theta, prefix, S, layout, n_slots):
        self.name, self.dt, self.theta, self.prefix, self.S = name, dt, theta, list(prefix), S
        self.B, self.Hq, self.Hkv, self.D = B, Hq, Hkv, D
        self.width = max(prefix) + S
        w = synth.Workload(name, B, Hq, Hkv, self.width, D, dt, theta, _seed(name))
        self.q_all, self.k_all, self.v_all = synth.make_inputs(w)
        self.q = torch.stack([self.q_all[b, p:p + S] for b, p in enumerate(prefix)]).contiguous()
        self.n_slots = n_slots
        self.map = _maps(layout, B, self.width, n_slots, _seed(name) + 1)
        self.kc = _garbage((n_slots, Hkv, D), dt, _seed(name) + 2)
        self.vc = _garbage((n_slots, Hkv, D), "bf16" if dt == "i16" else dt, _seed(name) + 3)
        for b, p in enumerate(prefix):
            slots = torch.from_numpy(self.map[b, :p + S].astype(np.int64))
            self.kc[slots] = self.k_all[b, :p + S]
            self.vc[slots] = self.v_all[b, :p + S]
        self.scale = _score_scale(dt, D)

    def oracle(self):
        f = synth.to_f64
        if self.dt == "i16":
            return oracle.attention_i16_cached(f(self.q), f(self.kc), f(self.vc), self.map, self.prefix,
                                               rope_theta=self.theta, score_scale=self.scale)
        return oracle.attention_cached(f(self.q), f(self.kc), f(self.vc), self.map, self.prefix,
                                       rope_theta=self.theta, scale=self.scale or None)

    def run(self, attn):
        dev = lambda t: t.cuda()  # noqa: E731
        off = torch.tensor(self.prefix, dtype=torch.int32, device="cuda")
        o = attn.run_cached(dev(self.q), dev(self.kc), dev(self.vc), dev(torch.from_numpy(self.map)),
                            pos_offsets=off, score_scale=self.scale)
        torch.cuda.synchronize()
        assert attn.status() == pa.PA_OK
        return o.cpu()


def _handle(c, max_seq=None):
    return pa.PrefillAttention(c.Hq, c.Hkv, c.D, max_seq or c.width, c.theta)


# ------------------------------------------------------------ cache update

@pytest.mark.parametrize("dt", ["f32", "bf16", "i16"])
def test_cache_update_is_bit_exact(dt):
    name = f"upd_{dt}"
    announce(name)
    B, S, Hkv, D, n_slots = 3, 37, 2, 128 if dt != "f32" else 64, 512
    prefix = [0, 5, 64]
    width = max(prefix) + S
    kv_map = _maps("paged", B, width, n_slots, _seed(name))
    kc = _garbage((n_slots, Hkv, D), dt, 1)
    vdt = "bf16" if dt == "i16" else dt
    vc = _garbage((n_slots, Hkv, D), vdt, 2)
    kn = _garbage((B, S, Hkv, D), dt, 3)
    vn = _garbage((B, S, Hkv, D), vdt, 4)
    attn = pa.PrefillAttention(4, Hkv, D, width, 1e4)
    try:
        kcd, vcd = kc.cuda(), vc.cuda()
        off = torch.tensor(prefix, dtype=torch.int32, device="cuda")
        attn.kv_cache_update(kn.cuda(), vn.cuda(), kcd, vcd, torch.from_numpy(kv_map).cuda(), off)
        torch.cuda.synchronize()
        assert attn.status() == pa.PA_OK
        bits = torch.int32 if dt == "f32" else torch.int16
        want_k, want_v = oracle.kv_cache_update(kc.view(bits).numpy(), vc.view(bits).numpy(), kn.view(bits).numpy(),
                                                vn.view(bits).numpy(), kv_map, prefix)
        assert np.array_equal(kcd.cpu().view(bits).numpy(), want_k)
        assert np.array_equal(vcd.cpu().view(bits).numpy(), want_v)
    finally:
        attn.close()


# ------------------------------------------------------------ cached == plain

PLAIN_CASES = [
    # name, B, Hq, Hkv, S, D, dtype, theta
    ("same_bf16_4wave", 1, 4, 2, 300, 128, "bf16", 1e4),
    ("same_bf16_8wave", 1, 64, 8, 1030, 96, "bf16", 1e4),
    ("same_bf16_8wave_paired", 1, 64, 8, 2000, 96, "bf16", 1e4),  # 256 pairs of query blocks
    ("same_bf16_8wave_d64", 1, 64, 64, 1030, 64, "bf16", 1e4),  # one head per workgroup
    ("same_bf16_8wave_d128", 1, 64, 16, 1030, 128, "bf16", 1e4),  # two-group schedule, four heads packed
    ("same_f32", 1, 2, 1, 200, 64, "f32", 1e4),
    ("same_i16", 1, 4, 4, 300, 128, "i16", 1e4),
]


@pytest.mark.parametrize("case", PLAIN_CASES, ids=[c[0] for c in PLAIN_CASES])
def test_identity_map_equals_plain_prefill_bitwise(case):
    name, B, Hq, Hkv, S, D, dt, theta = case
    announce(name)
    w = synth.Workload(name, B, Hq, Hkv, S, D, dt, theta, _seed(name), score_scale=_score_scale(dt, D))
    q, k, v = synth.make_inputs(w)
    attn = pa.PrefillAttention(Hq, Hkv, D, S, theta)
    try:
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        o_plain = attn(qd, kd, vd, score_scale=w.score_scale)
        ident = torch.arange(S, dtype=torch.int32, device="cuda")[None, :]
        o_cached = attn.run_cached(qd, kd[0], vd[0], ident, score_scale=w.score_scale)
        torch.cuda.synchronize()
        assert attn.status() == pa.PA_OK
        assert torch.equal(o_plain, o_cached)
    finally:
        attn.close()


# ------------------------------------------------------------ cached vs oracle

SMALL_CASES = [
    # name, B, Hq, Hkv, D, dtype, theta, prefix, S, layout, n_slots
    ("c_bf16_d64_ring", 2, 4, 2, 64, "bf16", 1e4, [0, 77], 150, "ring", 1024),
    ("c_bf16_d96_paged", 3, 4, 1, 96, "bf16", 1e4, [64, 300, 5], 129, "paged", 2048),
    ("c_bf16_d128_paged", 2, 8, 2, 128, "bf16", 1e6, [256, 1], 200, "paged", 1024),
    ("c_bf16_d128_decode_shape", 2, 4, 4, 128, "bf16", 1e4, [700, 1023], 1, "paged", 2048),
    ("c_f32_d64_paged", 2, 2, 1, 64, "f32", 1e4, [33, 128], 70, "paged", 512),
    ("c_f32_d128_ring", 1, 2, 2, 128, "f32", 1e4, [190], 66, "ring", 300),
    ("c_i16_d128_paged", 2, 4, 2, 128, "i16", 1e4, [100, 0], 160, "paged", 1024),
    ("c_i16_d64_ring", 1, 2, 1, 64, "i16", 1e4, [64], 64, "ring", 200),
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_cached_prefill_matches_oracle(case):
    c = Case(*case)
    announce(c.name)
    attn = _handle(c)
    try:
        got = c.run(attn)
    finally:
        attn.close()
    mx, mean = assert_close(got.numpy(), c.oracle(), "f32" if c.dt == "f32" else "bf16")
    announce(c.name, f"max {mx:.2e} mean {mean:.2e}")


# ------------------------------------------------------------ chunked pipelines

def _chunked(attn, q, k, v, chunks, kv_map, n_slots, dt, scale):
    """kv_cache_update + run_cached per chunk on device tensors; returns O [B][T][Hq][D]."""
    B, T, Hkv, D = k.shape
    kc = torch.zeros((n_slots, Hkv, D), dtype=k.dtype, device="cuda")
    vc = torch.zeros((n_slots, Hkv, D), dtype=v.dtype, device="cuda")
    mapd = torch.from_numpy(kv_map).cuda()
    outs, pos = [], 0
    for n in chunks:
        off = torch.full((B,), pos, dtype=torch.int32, device="cuda")
        attn.kv_cache_update(k[:, pos:pos + n].contiguous(), v[:, pos:pos + n].contiguous(), kc, vc, mapd, off)
        outs.append(attn.run_cached(q[:, pos:pos + n].contiguous(), kc, vc, mapd, pos_offsets=off, score_scale=scale))
        pos += n
    torch.cuda.synchronize()
    assert attn.status() == pa.PA_OK
    return torch.cat(outs, dim=1)


@pytest.mark.parametrize("name,B,Hq,Hkv,D,chunks", [
    ("chunk_8wave_d128", 4, 32, 8, 128, [512, 512, 512]),
    ("chunk_8wave_d96", 2, 32, 32, 96, [1024, 1024]),  # paired-barrier schedule at head_dim 96
    ("chunk_8wave_odd_tiles", 4, 32, 8, 128, [320, 704]),  # prefix 320: an odd count of whole tiles
    ("chunk_8wave_paired", 2, 64, 16, 96, [2048, 1024]),  # paired launches: two rounds, then one
    ("chunk_ragged_d64", 2, 8, 2, 64, [100, 333, 1, 250]),
])
def test_chunked_prefill_equals_plain_prefill(name, B, Hq, Hkv, D, chunks):
    T = sum(chunks)
    announce(name, chunks)
    w = synth.Workload(name, B, Hq, Hkv, T, D, "bf16", 1e4, _seed(name))
    q, k, v = synth.make_inputs(w)
    n_slots = B * ((T + 63) // 64) * 64 + 64
    kv_map = _maps("paged", B, T, n_slots, _seed(name), block=64)
    attn = pa.PrefillAttention(Hq, Hkv, D, T, 1e4)
    try:
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        o_chunk = _chunked(attn, qd, kd, vd, chunks, kv_map, n_slots, "bf16", 0.0).cpu()
        o_plain = attn(qd, kd, vd).cpu()
    finally:
        attn.close()
    # Chunk boundaries at multiples of 64 keep the same key tiles as the plain run.
    if all(n % 64 == 0 for n in chunks):
        assert torch.equal(o_chunk, o_plain)
    else:
        mx, _ = errors(o_chunk.numpy(), o_plain.numpy())
        assert mx <= 2e-3, mx
    rng = np.random.default_rng(3)
    rows = sorted({(int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(T))) for _ in range(48)}
                  | {(0, 0, 0), (B - 1, Hq - 1, T - 1)})
    want = oracle.attention_rows(q.float().numpy(), k.float().numpy(), v.float().numpy(), rows, rope_theta=1e4)
    got = np.stack([o_chunk[b, i, h].numpy() for b, h, i in rows])
    mx, _ = errors(got, want)
    assert mx <= 1e-2, mx


def test_long_prompt_in_four_chunks():
    """The 1 x 32 x 4096 x 96 long prompt, prefilled in chunks of 1024 through a
    ring cache: equal to the one-shot prefill, and to the oracle on sampled rows."""
    w = synth.WORKLOADS["mha_bf16_h32_s4096_d96"]
    announce(w.name, "chunks of 1024")
    q, k, v = synth.make_inputs(w)
    kv_map = oracle.ring_index_map(4096, 1000, 4096).astype(np.int32)[None, :]
    attn = pa.PrefillAttention(w.n_heads, w.n_kv_heads, w.head_dim, w.seq_len, w.rope_theta)
    try:
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        o_chunk = _chunked(attn, qd, kd, vd, [1024] * 4, kv_map, 4096, "bf16", 0.0).cpu()
        o_plain = attn(qd, kd, vd).cpu()
    finally:
        attn.close()
    assert torch.equal(o_chunk, o_plain)
    from gpu_common import oracle_rows, sample_rows
    rows = sample_rows(w, 64, seed=11)
    want = oracle_rows(w, q, k, v, rows)
    got = np.stack([o_chunk[b, i, h].numpy() for b, h, i in rows])
    mx, _ = errors(got, want)
    assert mx <= 1e-2, mx


# ------------------------------------------------------------ range errors

def test_bad_slot_is_read_as_slot_zero_and_reported():
    c = Case("bad_slot", 1, 2, 2, 64, "bf16", 1e4, [40], 30, "paged", 256)
    announce(c.name)
    attn = _handle(c)
    try:
        bad = c.map.copy()
        bad[0, 7] = c.n_slots + 5
        off = torch.tensor(c.prefix, dtype=torch.int32, device="cuda")
        o = attn.run_cached(c.q.cuda(), c.kc.cuda(), c.vc.cuda(), torch.from_numpy(bad).cuda(), pos_offsets=off)
        assert attn.status() == pa.PA_ERANGE
        assert torch.all(torch.isfinite(o))
        # the update skips the token whose slot is out of range
        kc, vc = c.kc.cuda(), c.vc.cuda()
        bad[0, 45] = -3
        kn = _garbage((1, 30, 2, 64), "bf16", 9).cuda()
        attn.kv_cache_update(kn, kn, kc, vc, torch.from_numpy(bad).cuda(), off)
        assert attn.status() == pa.PA_ERANGE
        slots = bad[0, 40:70]
        for i, s in enumerate(slots):
            if 0 <= s < c.n_slots:
                assert torch.equal(kc[s].cpu(), kn[0, i].cpu())
    finally:
        attn.close()


# name, B, Hq, Hkv, D, dtype, prefix, S, n_split: the four-wave kernels (bf16 and
# int16), the paired eight-wave kernel at head_dim 96, the two-group one at 128
# (heads packed four to a workgroup), and an eight-wave split launch
DEEP_BAD = [
    ("deep_bad_4wave_d64", 1, 2, 2, 64, "bf16", 1100, 40, 1),
    ("deep_bad_4wave_i16_d64", 1, 2, 2, 64, "i16", 1100, 40, 1),
    ("deep_bad_8wave_d96", 8, 32, 32, 96, "bf16", 1100, 256, 1),
    ("deep_bad_8wave_d128", 8, 32, 8, 128, "bf16", 1100, 256, 1),
    ("deep_bad_split_d96", 1, 32, 32, 96, "bf16", 1100, 256, 8),
]


@pytest.mark.parametrize("case", DEEP_BAD, ids=[c[0] for c in DEEP_BAD])
def test_bad_slots_deep_in_the_prefix_read_slot_zero(case):
    """Map entries outside the cache at keys that the key loop (not the
    prologue) stages, in the prefix and in the chunk: the run reads slot 0 for
    them and reports the range error, so its O equals bit for bit that of a
    run whose map holds slot 0 at those keys (which reports nothing)."""
    name, B, Hq, Hkv, D, dt, prefix, S, n_split = case
    width = prefix + S
    n_slots = B * ((width + 63) // 64) * 64 + 64
    c = Case(name, B, Hq, Hkv, D, dt, 1e4, [prefix] * B, S, "paged", n_slots)
    announce(c.name, "n_split", n_split)
    bad, zero = c.map.copy(), c.map.copy()
    keys = [5, 700, 701, prefix - 1, prefix + 10]
    for i, j in enumerate(keys):
        bad[B - 1, j] = n_slots + i if i % 2 == 0 else -1 - i
        zero[B - 1, j] = 0
    attn = _handle(c)
    try:
        off = torch.tensor(c.prefix, dtype=torch.int32, device="cuda")
        qd, kcd, vcd = c.q.cuda(), c.kc.cuda(), c.vc.cuda()
        ws = None
        if n_split > 1:
            ws = torch.empty(pa.prefill_attn_run_cached_workspace_size(attn.handle, B, S, n_split),
                             dtype=torch.uint8, device="cuda")
        outs, codes = [], []
        for m in (bad, zero):
            o = attn.run_cached(qd, kcd, vcd, torch.from_numpy(m).cuda(), pos_offsets=off, score_scale=c.scale,
                                n_split=n_split, workspace=ws)
            torch.cuda.synchronize()
            codes.append(attn.status())
            outs.append(o.cpu())
    finally:
        attn.close()
    assert codes == [pa.PA_ERANGE, pa.PA_OK], codes
    assert torch.isfinite(outs[0]).all()
    assert torch.equal(outs[0], outs[1])


def test_chunk_past_the_map_row_zeroes_that_sequence():
    c = Case("short_map", 2, 2, 1, 64, "bf16", 1e4, [10, 20], 40, "paged", 512)
    announce(c.name)
    attn = _handle(c, max_seq=256)
    try:
        off = torch.tensor([10, 30], dtype=torch.int32, device="cuda")  # 30 + 40 > map_stride 60
        out = torch.full(c.q.shape, 7.0, dtype=torch.float32, device="cuda")
        attn.run_cached(c.q.cuda(), c.kc.cuda(), c.vc.cuda(), torch.from_numpy(c.map).cuda(), pos_offsets=off,
                        out=out)
        assert attn.status() == pa.PA_ERANGE
        o = out.cpu()
        assert torch.all(o[1] == 0)
        assert torch.all(torch.isfinite(o[0])) and not torch.all(o[0] == 7.0)
    finally:
        attn.close()


def test_cache_calls_reject_bad_arguments():
    attn = pa.PrefillAttention(2, 2, 64, 64, 1e4)
    lib = pa.load_library()
    try:
        buf = torch.zeros(1 << 16, dtype=torch.float32, device="cuda")
        p = buf.data_ptr()
        h = attn.handle
        s = torch.cuda.current_stream().cuda_stream
        run = lambda *a: lib.prefill_attn_run_cached(h, *a)  # noqa: E731
        upd = lambda *a: lib.prefill_attn_kv_cache_update(h, *a)  # noqa: E731
        assert run(pa.PA_IN_BF16, 1, 8, p, p, p, 0, p, 8, None, p, 0.0, s) == pa.PA_EINVAL    # no slots
        assert run(pa.PA_IN_BF16, 1, 8, p, p, p, 16, p, 4, None, p, 0.0, s) == pa.PA_EINVAL   # map row < chunk
        assert run(pa.PA_IN_BF16, 1, 8, p, p, p, 16, None, 8, None, p, 0.0, s) == pa.PA_EINVAL  # no map
        assert run(pa.PA_IN_BF16, 1, 8, p, p, p, 16, p + 2, 8, None, p, 0.0, s) == pa.PA_EINVAL  # misaligned map
        assert run(pa.PA_IN_BF16, 1, 8, p, p + 8, p, 16, p, 8, None, p, 0.0, s) == pa.PA_EINVAL  # misaligned cache
        assert run(pa.PA_IN_BF16, 1, 8, p, p, p, 1 << 24, p, 8, None, p, 0.0, s) == pa.PA_EINVAL  # cache > 4 GiB
        assert run(9, 1, 8, p, p, p, 16, p, 8, None, p, 0.0, s) == pa.PA_EINVAL
        assert upd(pa.PA_IN_BF16, 1, 8, p, p, None, p, 4, p, p, 16, s) == pa.PA_EINVAL
        assert upd(pa.PA_IN_BF16, 1, 8, p, None, None, p, 8, p, p, 16, s) == pa.PA_EINVAL
        assert upd(pa.PA_IN_BF16, 0, 8, None, None, None, None, 8, None, None, 16, s) == pa.PA_OK
        torch.cuda.synchronize()
        assert attn.status() == pa.PA_OK
    finally:
        attn.close()


# ------------------------------------------------------------ split-K cached prefill

# Split and unsplit runs round P~ to fp16 against different running maxima:
# each element may differ by two half-ulps, 2^-10 relative, times |V| up to
# ~4 in these workloads (per-head scales up to 2, 2 sigma) -> 4e-3 max-abs.
# Far below the oracle bars, which both runs must meet on their own.
SPLIT_TOL_MAX = 4e-3
SPLIT_TOL_MEAN = 1e-4  # a key dropped from a 2000-key row moves O by ~5e-4 on average

SPLIT_CASES = [
    # name, B, Hq, Hkv, D, dtype, theta, prefix, S, layout, n_slots, n_split
    ("sk_bf16_d128_paged", 2, 8, 2, 128, "bf16", 1e4, [700, 1300], 150, "paged", 4096, 4),
    ("sk_bf16_d96_ring_auto", 1, 4, 4, 96, "bf16", 1e4, [2000], 100, "ring", 4096, 0),
    ("sk_bf16_d64_many", 2, 4, 2, 64, "bf16", 1e4, [64, 5], 77, "paged", 1024, 9),
    ("sk_i16_d128", 1, 4, 2, 128, "i16", 1e4, [900], 128, "paged", 2048, 3),
    ("sk_bf16_d128_8wave", 1, 32, 8, 128, "bf16", 1e4, [1500], 256, "paged", 2048, 8),  # two-group split
    # Rows (B * S * Hq) not a multiple of the merge's rows per workgroup
    # (10 at head_dim 96, 8 at 128): the last merge workgroup is partial.
    ("sk_bf16_d96_merge_tail", 1, 3, 1, 96, "bf16", 1e4, [1300], 37, "paged", 2048, 5),
    ("sk_bf16_d128_merge_tail", 1, 5, 1, 128, "bf16", 1e4, [611], 45, "ring", 1024, 3),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_split_k_cached_prefill(case):
    """Split-K partials merged by the log-sum-exp rule: against the oracle at the
    usual bars, and against the unsplit cached run (they differ only through the
    fp16 rounding of P~ relative to each split's running max)."""
    *head, n_split = case
    c = Case(*head)
    announce(c.name, "n_split", n_split)
    attn = _handle(c)
    try:
        off = torch.tensor(c.prefix, dtype=torch.int32, device="cuda")
        qd, kcd, vcd, mapd = c.q.cuda(), c.kc.cuda(), c.vc.cuda(), torch.from_numpy(c.map).cuda()
        ws = torch.empty(pa.prefill_attn_run_cached_workspace_size(attn.handle, c.B, c.S, 16), dtype=torch.uint8,
                         device="cuda")
        o_split = attn.run_cached(qd, kcd, vcd, mapd, pos_offsets=off, score_scale=c.scale, n_split=n_split,
                                  workspace=ws)
        o_one = attn.run_cached(qd, kcd, vcd, mapd, pos_offsets=off, score_scale=c.scale)
        torch.cuda.synchronize()
        assert attn.status() == pa.PA_OK
        o_split, o_one = o_split.cpu(), o_one.cpu()
    finally:
        attn.close()
    mx, mean = errors(o_split.numpy(), o_one.numpy())
    assert mx <= SPLIT_TOL_MAX and mean <= SPLIT_TOL_MEAN, f"split vs unsplit {mx:.3e} / {mean:.3e}"
    mx, mean = assert_close(o_split.numpy(), c.oracle(), "bf16")
    announce(c.name, f"max {mx:.2e} mean {mean:.2e}")


def test_split_k_long_prompt_chunks():
    """The 1 x 32 x 4096 x 96 long prompt in chunks of 1024 with split-K against
    the one-shot prefill (merge rounding only) and the oracle on sampled rows."""
    w = synth.WORKLOADS["mha_bf16_h32_s4096_d96"]
    announce(w.name, "chunks of 1024, split-K")
    q, k, v = synth.make_inputs(w)
    kv_map = torch.from_numpy(oracle.ring_index_map(4096, 1000, 4096).astype(np.int32)[None, :]).cuda()
    attn = pa.PrefillAttention(w.n_heads, w.n_kv_heads, w.head_dim, w.seq_len, w.rope_theta)
    try:
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        kc = torch.zeros((4096, 32, 96), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        ws = torch.empty(pa.prefill_attn_run_cached_workspace_size(attn.handle, 1, 1024, 8), dtype=torch.uint8,
                         device="cuda")
        outs = []
        for p in range(0, 4096, 1024):
            off = torch.tensor([p], dtype=torch.int32, device="cuda")
            attn.kv_cache_update(kd[:, p:p + 1024].contiguous(), vd[:, p:p + 1024].contiguous(), kc, vc, kv_map, off)
            outs.append(attn.run_cached(qd[:, p:p + 1024].contiguous(), kc, vc, kv_map, pos_offsets=off, n_split=0,
                                        workspace=ws))
        o_chunk = torch.cat(outs, dim=1).cpu()
        o_plain = attn(qd, kd, vd).cpu()
        assert attn.status() == pa.PA_OK
    finally:
        attn.close()
    mx, mean = errors(o_chunk.numpy(), o_plain.numpy())
    assert mx <= SPLIT_TOL_MAX and mean <= SPLIT_TOL_MEAN, (mx, mean)
    from gpu_common import oracle_rows, sample_rows
    rows = sample_rows(w, 48, seed=12)
    got = np.stack([o_chunk[b, i, h].numpy() for b, h, i in rows])
    mx, _ = errors(got, oracle_rows(w, q, k, v, rows))
    assert mx <= 1e-2, mx


def test_split_k_range_error_gives_zeros():
    c = Case("sk_range", 2, 2, 1, 64, "bf16", 1e4, [10, 20], 40, "paged", 512)
    announce(c.name)
    attn = _handle(c, max_seq=256)
    try:
        off = torch.tensor([10, 30], dtype=torch.int32, device="cuda")  # 30 + 40 > map_stride 60
        out = torch.full(c.q.shape, 7.0, dtype=torch.float32, device="cuda")
        ws = torch.empty(pa.prefill_attn_run_cached_workspace_size(attn.handle, 2, 40, 4), dtype=torch.uint8,
                         device="cuda")
        attn.run_cached(c.q.cuda(), c.kc.cuda(), c.vc.cuda(), torch.from_numpy(c.map).cuda(), pos_offsets=off,
                        out=out, n_split=4, workspace=ws)
        assert attn.status() == pa.PA_ERANGE
        o = out.cpu()
        assert torch.all(o[1] == 0)
        assert torch.all(torch.isfinite(o[0])) and not torch.all(o[0] == 7.0)
    finally:
        attn.close()


# ------------------------------------------------------------ update fused into the attention launch

FUSED_CASES = [
    # name, B, Hq, Hkv, D, dtype (bf16q: bf16 quantised in-kernel), chunks, layout, n_split
    ("fu_bf16_d96_8wave", 1, 32, 32, 96, "bf16", [1024, 1024, 512], "ring", 0),
    ("fu_bf16_d128_gqa_split", 2, 16, 4, 128, "bf16", [300, 700, 64], "paged", 4),
    ("fu_bf16_d96_gqa2_8wave", 2, 32, 16, 96, "bf16", [300, 77, 513], "ring", 0),  # two heads per workgroup
    ("fu_bf16_d64_4wave", 2, 4, 2, 64, "bf16", [100, 333, 1, 250], "paged", 1),
    ("fu_i16_d128", 1, 8, 2, 128, "i16", [200, 456], "ring", 1),
    ("fu_i16_d128_split", 1, 8, 2, 128, "i16", [512, 300], "paged", 3),
    ("fu_q16_d96", 1, 4, 4, 96, "bf16q", [130, 290], "ring", 0),
    ("fu_f32_d64", 1, 2, 2, 64, "f32", [70, 90], "paged", 1),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_run_cached_update_equals_update_then_run(case):
    """prefill_attn_run_cached_update on each chunk against kv_cache_update then
    run_cached(_splitk) on a copy of the same cache: every output and the final
    caches bit for bit."""
    name, B, Hq, Hkv, D, dt, chunks, layout, n_split = case
    T = sum(chunks)
    announce(name, chunks, "split", n_split)
    w = synth.Workload(name, B, Hq, Hkv, T, D, dt, 1e4, _seed(name))
    q, k, v = synth.make_inputs(w)
    n_slots = B * ((T + 63) // 64) * 64 + 64
    kv_map = _maps(layout, B, T, n_slots, _seed(name), block=64)
    quant = dt == "bf16q"
    scale = _score_scale(dt, D)
    attn = pa.PrefillAttention(Hq, Hkv, D, T, 1e4)
    try:
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        mapd = torch.from_numpy(kv_map).cuda()
        caches = [(_garbage((n_slots, Hkv, D), "i16" if dt == "i16" else "bf16" if dt != "f32" else "f32", 7),
                   _garbage((n_slots, Hkv, D), "f32" if dt == "f32" else "bf16", 8)) for _ in range(2)]
        (kc1, vc1), (kc2, vc2) = [(a.cuda(), b.cuda()) for a, b in caches]
        ws_bytes = pa.prefill_attn_run_cached_workspace_size(attn.handle, B, max(chunks), 16)
        ws1 = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        ws2 = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        pos = 0
        for n in chunks:
            off = torch.full((B,), pos, dtype=torch.int32, device="cuda")
            qc, kn, vn = (x[:, pos:pos + n].contiguous() for x in (qd, kd, vd))
            attn.kv_cache_update(kn, vn, kc1, vc1, mapd, off)
            o1 = attn.run_cached(qc, kc1, vc1, mapd, pos_offsets=off, score_scale=scale, quantize=quant,
                                 n_split=n_split, workspace=ws1 if n_split != 1 else None)
            o2 = attn.run_cached_update(qc, kn, vn, kc2, vc2, mapd, pos_offsets=off, score_scale=scale,
                                        quantize=quant, n_split=n_split, workspace=ws2 if n_split != 1 else None)
            torch.cuda.synchronize()
            assert attn.status() == pa.PA_OK
            assert torch.equal(o1, o2), f"chunk at {pos}: max diff {float((o1 - o2).abs().max()):.3e}"
            pos += n
        assert torch.equal(kc1, kc2) and torch.equal(vc1, vc2)
    finally:
        attn.close()


def test_run_cached_update_bad_slot_is_skipped_and_reported():
    """A map entry outside the cache for one of the chunk's own tokens: that row is
    not written (the rest are), and the status word reads PA_ERANGE."""
    B, Hq, Hkv, D, S = 1, 2, 2, 64, 100
    w = synth.Workload("fu_bad_slot", B, Hq, Hkv, S, D, "bf16", 1e4, 91)
    q, k, v = synth.make_inputs(w)
    n_slots = 128
    kv_map = np.arange(S, dtype=np.int32)[None, :].copy()
    kv_map[0, 37] = n_slots + 5
    attn = pa.PrefillAttention(Hq, Hkv, D, S, 1e4)
    try:
        kc = torch.zeros((n_slots, Hkv, D), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        attn.run_cached_update(q.cuda(), k.cuda(), v.cuda(), kc, vc, torch.from_numpy(kv_map).cuda())
        torch.cuda.synchronize()
        assert attn.status() == pa.PA_ERANGE
        kc, vc = kc.cpu(), vc.cpu()
        rows = [i for i in range(S) if i != 37]
        assert torch.equal(kc[rows], k[0, rows]) and torch.equal(vc[rows], v[0, rows])
        assert torch.all(kc[S:] == 0)
    finally:
        attn.close()
