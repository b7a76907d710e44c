"""GPU test of prefill_attn_decode_noalloc, the decode call whose split partials
live in the library's fixed device scratch instead of a caller workspace.

Through the C-ABI: its output must equal prefill_attn_decode's with a
workspace and the same split, bit for bit (the same kernels run on the same
partials), on two calls in a row, the second with a smaller input, so that the
second call runs over scratch that the first one left behind.  The first call
is also held to the decode tolerance against the fp64 oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import rope_causal_attention_amd as pa
import synth
from gpu_common import announce, errors, need_gpu

pytestmark = pytest.mark.gpu

TOL = 1e-5  # decode computes in fp32


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _case(seed, B, Hq, Hkv, D, pos, block=16):
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    width = max(pos) + 1
    need = (width + block - 1) // block
    n_blocks = B * need + 1
    perm = rng.permutation(n_blocks)
    kv_map = np.stack([oracle.paged_index_map(perm[b * need:(b + 1) * need], block, width)
                       for b in range(B)]).astype(np.int32)
    n_slots = n_blocks * block
    kc = torch.randn((n_slots, Hkv, D), generator=g).bfloat16()
    vc = torch.randn((n_slots, Hkv, D), generator=g).bfloat16()
    q = (torch.randn((B, Hq, D), generator=g) * 1.5).bfloat16()
    return q, kc, vc, kv_map, n_slots


def _both(attn, q, kc, vc, kv_map, n_slots, pos, n_split):
    """(noalloc output, workspace output) for the same call."""
    B, Hq, D = q.shape
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    md = torch.from_numpy(kv_map).cuda()
    off = torch.tensor(pos, dtype=torch.int32, device="cuda")
    o_na = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    o_ws = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    pa.prefill_attn_decode_noalloc(attn.handle, pa.PA_IN_BF16, B, qd, kd, vd, n_slots, md, kv_map.shape[1], off,
                                   o_na, 0.0, n_split)
    ws_bytes = pa.prefill_attn_decode_workspace_size(attn.handle, B, 1024)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    pa.prefill_attn_decode(attn.handle, pa.PA_IN_BF16, B, qd, kd, vd, n_slots, md, kv_map.shape[1], off, o_ws, 0.0,
                           n_split, ws, ws_bytes)
    torch.cuda.synchronize()
    assert attn.status() == pa.PA_OK
    return o_na.cpu(), o_ws.cpu()


def test_noalloc_decode_equals_workspace_decode_twice():
    Hq, Hkv, D = 32, 8, 128
    attn = pa.PrefillAttention(Hq, Hkv, D, 4096, 1e4)
    try:
        # first call: 8 sequences, explicit 6-way split (0.8 MB of partials in the 8 MiB scratch)
        pos1 = [4095, 3000, 17, 2048, 4000, 999, 1, 3500]
        q, kc, vc, kv_map, n_slots = _case(11, 8, Hq, Hkv, D, pos1)
        assert pa.prefill_attn_decode_workspace_size(attn.handle, 8, 6) <= pa.prefill_attn_decode_noalloc_scratch_bytes()
        announce("noalloc first call", "B", 8, "split", 6)
        got, ref = _both(attn, q, kc, vc, kv_map, n_slots, pos1, 6)
        assert torch.equal(got, ref)
        f = synth.to_f64
        for b in (0, 2, 6):
            want = oracle.attention_cached(f(q[b:b + 1])[:, None], f(kc), f(vc), kv_map[b:b + 1], [pos1[b]],
                                           rope_theta=1e4)[:, 0]
            mx, _ = errors(got[b:b + 1].numpy(), want)
            assert mx <= TOL, (b, mx)

        # second call: a smaller input over the scratch the first call left, split chosen by the library
        pos2 = [700, 33]
        q2, kc2, vc2, map2, n_slots2 = _case(12, 2, Hq, Hkv, D, pos2)
        announce("noalloc second call", "B", 2, "split", "auto")
        got2, ref2 = _both(attn, q2, kc2, vc2, map2, n_slots2, pos2, 0)
        assert torch.equal(got2, ref2)
        assert torch.isfinite(got2).all()
    finally:
        attn.close()


def test_noalloc_decode_rejects_a_split_beyond_the_scratch():
    Hq, Hkv, D, B = 32, 8, 128, 64
    attn = pa.PrefillAttention(Hq, Hkv, D, 512, 1e4)
    try:
        pos = [300] * B
        q, kc, vc, kv_map, n_slots = _case(13, B, Hq, Hkv, D, pos)
        assert pa.prefill_attn_decode_workspace_size(attn.handle, B, 8) > pa.prefill_attn_decode_noalloc_scratch_bytes()
        announce("noalloc too big", "B", B, "split", 8)
        o = torch.zeros((B, Hq, D), dtype=torch.float32, device="cuda")
        with pytest.raises(pa.PrefillAttnError) as err:
            pa.prefill_attn_decode_noalloc(attn.handle, pa.PA_IN_BF16, B, q.cuda(), kc.cuda(), vc.cuda(), n_slots,
                                           torch.from_numpy(kv_map).cuda(), kv_map.shape[1],
                                           torch.tensor(pos, dtype=torch.int32, device="cuda"), o, 0.0, 8)
        assert err.value.code == pa.PA_ETOOBIG
        torch.cuda.synchronize()
        assert torch.all(o == 0)  # nothing was enqueued
    finally:
        attn.close()
