"""The library's calls under HIP graph capture.

prefill_attn_run and prefill_attn_decode_noalloc only launch kernels on the
caller's stream (no allocation, no memset, no synchronisation), so a caller
may capture them into a graph and replay it.  Each case captures one call on
fixed buffers, then replays the graph several times with new input values
copied into those buffers between replays (eager work and a synchronisation
in between), and checks every replay bit for bit against an eager call on the
same inputs.
"""

import numpy as np
import pytest
import torch

import oracle
import rope_causal_attention_amd as pa
import synth
from gpu_common import announce, need_gpu

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


# name, H, Hkv, S, D: a four-wave launch, and an eight-wave one (two-group schedule at 128)
SHAPES = [("graph_run_4wave_d96", 8, 2, 777, 96), ("graph_run_8wave_d128", 32, 8, 2048, 128)]


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_prefill_run_in_a_graph(shape):
    name, H, Hkv, S, D = shape
    announce(name)
    attn = pa.PrefillAttention(H, Hkv, D, S, 1e4)
    try:
        draws = [synth.make_inputs(synth.Workload(name, 1, H, Hkv, S, D, "bf16", 1e4, 7000 + r))
                 for r in range(REPLAYS + 1)]
        q, k, v = (t.cuda() for t in draws[0])
        out = torch.empty((1, S, H, D), dtype=torch.float32, device="cuda")
        g = _capture(lambda: attn(q, k, v, out=out))
        for r in range(1, REPLAYS + 1):
            for dst, src in zip((q, k, v), draws[r]):
                dst.copy_(src)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            want = attn(q, k, v)
            torch.cuda.synchronize()
            assert torch.equal(out, want), f"replay {r}"
        assert attn.status() == pa.PA_OK
    finally:
        attn.close()


def test_noalloc_decode_in_a_graph():
    B, Hq, Hkv, D, block = 4, 32, 8, 128, 16
    pos = [3000, 17, 1024, 2047]
    announce("graph_decode_noalloc")
    rng = np.random.default_rng(7100)
    width = max(pos) + 1
    need = (width + block - 1) // block
    n_blocks = B * need + 1
    perm = rng.permutation(n_blocks)
    kv_map = np.stack([oracle.paged_index_map(perm[b * need:(b + 1) * need], block, width)
                       for b in range(B)]).astype(np.int32)
    n_slots = n_blocks * block
    gen = torch.Generator().manual_seed(7100)
    kc = torch.randn((n_slots, Hkv, D), generator=gen).bfloat16().cuda()
    vc = torch.randn((n_slots, Hkv, D), generator=gen).bfloat16().cuda()
    qs = [(torch.randn((B, Hq, D), generator=gen) * 1.5).bfloat16() for _ in range(REPLAYS + 1)]
    md = torch.from_numpy(kv_map).cuda()
    off = torch.tensor(pos, dtype=torch.int32, device="cuda")
    attn = pa.PrefillAttention(Hq, Hkv, D, width, 1e4)
    try:
        q = qs[0].cuda()
        out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")

        def call(o):
            pa.prefill_attn_decode_noalloc(attn.handle, pa.PA_IN_BF16, B, q, kc, vc, n_slots, md, width, off,
                                           o, 0.0, 8)

        g = _capture(lambda: call(out))
        for r in range(1, REPLAYS + 1):
            q.copy_(qs[r])
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            want = torch.empty_like(out)
            call(want)
            torch.cuda.synchronize()
            assert torch.equal(out, want), f"replay {r}"
        assert attn.status() == pa.PA_OK
    finally:
        attn.close()
