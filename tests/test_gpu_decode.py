"""GPU parity of decode attention (one new token per sequence against the KV
cache) through the C-ABI, against the fp64 oracle.

Decode is the cached prefill of a one-token chunk, so the oracle is
``oracle.attention_cached`` with seq_len = 1.  The kernel computes in fp32
throughout (bf16 inputs are widened exactly), so every case is held to the
fp32 tolerance: max-abs 1e-5 over the whole output.
"""

import numpy as np
import pytest
import torch

import oracle
import rope_causal_attention_amd as pa
import synth
from gpu_common import announce, errors, need_gpu

pytestmark = pytest.mark.gpu

TOL = 1e-5
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _seed(name):
    return sum(map(ord, name))


class Decode:
    """Sequences of lengths pos[b] + 1 scattered over a paged cache, and the new
    tokens' queries."""

    def __init__(self, name, B, Hq, Hkv, D, dt, pos, theta=1e4, block=16, spare=2):
        self.name, self.B, self.Hq, self.Hkv, self.D, self.dt, self.pos, self.theta = \
            name, B, Hq, Hkv, D, dt, list(pos), theta
        g = torch.Generator().manual_seed(_seed(name))
        width = max(pos) + 1
        need = (width + block - 1) // block
        n_blocks = B * need + spare
        self.n_slots = n_blocks * block
        rng = np.random.default_rng(_seed(name))
        perm = rng.permutation(n_blocks)
        self.map = np.stack([oracle.paged_index_map(perm[b * need:(b + 1) * need], block, width)
                             for b in range(B)]).astype(np.int32)
        self.kc = (torch.randn((self.n_slots, Hkv, D), generator=g)).to(TORCH_DT[dt])
        self.vc = (torch.randn((self.n_slots, Hkv, D), generator=g)).to(TORCH_DT[dt])
        self.q = (torch.randn((B, Hq, D), generator=g) * 1.5).to(TORCH_DT[dt])

    def oracle(self):
        f = synth.to_f64
        return oracle.attention_cached(f(self.q)[:, None], f(self.kc), f(self.vc), self.map, self.pos,
                                       rope_theta=self.theta)[:, 0]

    def run(self, n_split=0, ws_bytes=None, expect=pa.PA_OK):
        attn = pa.PrefillAttention(self.Hq, self.Hkv, self.D, max(self.pos) + 1, self.theta)
        try:
            ws = None
            if ws_bytes is None:
                ws_bytes = pa.prefill_attn_decode_workspace_size(attn.handle, self.B, max(n_split, 64))
            if ws_bytes:
                ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
            off = torch.tensor(self.pos, dtype=torch.int32, device="cuda")
            o = attn.decode(self.q.cuda(), self.kc.cuda(), self.vc.cuda(), torch.from_numpy(self.map).cuda(),
                            pos_offsets=off, n_split=n_split, workspace=ws)
            torch.cuda.synchronize()
            assert attn.status() == expect
            return o.cpu()
        finally:
            attn.close()


CASES = [
    # name, B, Hq, Hkv, D, dtype, positions
    ("dec_gqa4_d128_bf16", 3, 32, 8, 128, "bf16", [0, 100, 1000]),
    ("dec_gqa4_d128_f32", 3, 32, 8, 128, "f32", [5, 777, 64]),
    ("dec_mha_d64_bf16", 2, 4, 4, 64, "bf16", [300, 17]),
    ("dec_gqa2_d96_bf16", 2, 8, 4, 96, "bf16", [511, 512]),
    ("dec_gqa8_d128_bf16", 2, 16, 2, 128, "bf16", [2047, 1]),
    ("dec_gqa16_d64_f32", 1, 32, 2, 64, "f32", [900]),
    ("dec_gqa6_d96_f32", 2, 12, 2, 96, "f32", [250, 3]),
    ("dec_gqa3_d128_bf16", 2, 6, 2, 128, "bf16", [129, 40]),
]


@pytest.mark.parametrize("n_split", [1, 0, 7])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_matches_oracle(case, n_split):
    c = Decode(*case)
    announce(c.name, "split", n_split)
    got = c.run(n_split=n_split)
    mx, mean = errors(got.numpy(), c.oracle())
    announce(c.name, f"max {mx:.2e} mean {mean:.2e}")
    assert mx <= TOL, mx


def test_more_splits_than_keys():
    c = Decode("dec_tiny", 2, 4, 2, 64, "bf16", [0, 3])
    announce(c.name)
    mx, _ = errors(c.run(n_split=16).numpy(), c.oracle())
    assert mx <= TOL, mx


def test_small_workspace_falls_back_to_fewer_splits():
    c = Decode("dec_ws", 2, 8, 2, 128, "bf16", [3000, 1500])
    announce(c.name)
    want = c.oracle()
    for ws in (0, 100, 2 * 8 * 4 * (128 + 2) * 4):  # none, too small for 2 splits, room for 4
        mx, _ = errors(c.run(n_split=12, ws_bytes=ws).numpy(), want)
        assert mx <= TOL, (ws, mx)


def test_long_context_batch():
    """16 sequences of up to 4096 cached tokens, 32 query / 8 KV heads, D = 128."""
    pos = [4095, 4000, 3500, 4095, 2048, 1024, 4095, 3333, 100, 4095, 2999, 4095, 4094, 1, 4095, 3900]
    c = Decode("dec_long", 16, 32, 8, 128, "bf16", pos, block=64)
    announce(c.name)
    got = c.run()
    f = synth.to_f64
    for b in (0, 4, 8, 13, 15):
        want = oracle.attention_cached(f(c.q[b:b + 1])[:, None], f(c.kc), f(c.vc), c.map[b:b + 1], [pos[b]])[:, 0]
        mx, _ = errors(got[b:b + 1].numpy(), want)
        assert mx <= TOL, (b, mx)


def test_positions_outside_the_table_or_map_give_zeros():
    c = Decode("dec_range", 3, 4, 2, 64, "bf16", [10, 20, 30])
    announce(c.name)
    attn = pa.PrefillAttention(4, 2, 64, 31, 1e4)
    try:
        off = torch.tensor([10, 31, -1], dtype=torch.int32, device="cuda")  # 31 + 1 > max_seq, -1 < 0
        o = attn.decode(c.q.cuda(), c.kc.cuda(), c.vc.cuda(), torch.from_numpy(c.map).cuda(), pos_offsets=off,
                        n_split=1)
        assert attn.status() == pa.PA_ERANGE
        o = o.cpu()
        assert torch.all(o[1:] == 0) and not torch.all(o[0] == 0)
    finally:
        attn.close()


def test_bad_slot_is_reported():
    c = Decode("dec_badslot", 1, 4, 2, 64, "f32", [50])
    announce(c.name)
    c.map[0, 7] = c.n_slots + 3
    got = c.run(n_split=1, expect=pa.PA_ERANGE)
    assert torch.all(torch.isfinite(got))


def test_decode_rejects_bad_arguments():
    attn = pa.PrefillAttention(4, 2, 64, 64, 1e4)
    lib = pa.load_library()
    try:
        buf = torch.zeros(1 << 16, dtype=torch.float32, device="cuda")
        p = buf.data_ptr()
        h = attn.handle
        s = torch.cuda.current_stream().cuda_stream
        dec = lambda *a: lib.prefill_attn_decode(h, *a)  # noqa: E731
        assert dec(pa.PA_IN_I16, 1, p, p, p, 16, p, 8, None, p, 0.0, 0, None, 0, s) == pa.PA_EINVAL  # no int16
        assert dec(pa.PA_IN_BF16, 1, p, p, p, 0, p, 8, None, p, 0.0, 0, None, 0, s) == pa.PA_EINVAL   # no slots
        assert dec(pa.PA_IN_BF16, 1, p + 4, p, p, 16, p, 8, None, p, 0.0, 0, None, 0, s) == pa.PA_EINVAL
        assert dec(pa.PA_IN_BF16, 1, p, p, p, 16, None, 8, None, p, 0.0, 0, None, 0, s) == pa.PA_EINVAL
        assert dec(pa.PA_IN_BF16, 1, p, p, p, 16, p, 8, None, p, 0.0, -1, None, 0, s) == pa.PA_EINVAL
        assert dec(pa.PA_IN_BF16, 1, p, p, p, 16, p, 8, None, p, 0.0, 4, p + 8, 1 << 20, s) == pa.PA_EINVAL
        assert dec(pa.PA_IN_BF16, 0, None, None, None, 16, None, 8, None, None, 0.0, 0, None, 0, s) == pa.PA_OK
        torch.cuda.synchronize()
        assert attn.status() == pa.PA_OK
    finally:
        attn.close()
