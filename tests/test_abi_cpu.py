"""C-ABI checks that need no GPU: the library loads, exports what the header
declares, its host RoPE table builder agrees bit-for-bit with the oracle's
independently written tables, and argument errors come back as status codes.
"""

import math
import os
import re

import numpy as np
import pytest
import torch

import oracle
import rope_causal_attention_amd as pa
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "prefill_attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(prefill_attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = pa.load_library()
    declared = _declared_functions()
    assert declared, "no declarations parsed"
    assert sorted(pa.EXPORTED_SYMBOLS) == declared
    for name in declared:
        assert hasattr(lib, name), name


def test_single_hip_runtime_in_process():
    pa.load_library()
    maps = [l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l]
    assert len({os.path.realpath(p) for p in maps}) <= 1


@pytest.mark.parametrize("max_seq,D,theta", [(64, 64, 1e4), (4096, 96, 1e4), (512, 128, 1e6), (33, 2, 500.0)])
def test_f32_table_matches_oracle_bitwise(max_seq, D, theta):
    t = pa.prefill_attn_rope_table_f32(max_seq, D, theta)
    cos, sin = oracle.rope_cos_sin(np.arange(max_seq), D, theta)
    assert np.array_equal(t[..., 0], cos.astype(np.float32))
    assert np.array_equal(t[..., 1], sin.astype(np.float32))


@pytest.mark.parametrize("max_seq,D,theta", [(2048, 128, 1e4), (300, 96, 1e6), (64, 64, 1e4)])
def test_q14_table_matches_oracle_bitwise(max_seq, D, theta):
    t = pa.prefill_attn_rope_table_q14(max_seq, D, theta)
    C, S = oracle.rope_table_q14(max_seq, D, theta)
    assert np.array_equal(t[..., 0].astype(np.int64), C)
    assert np.array_equal(t[..., 1].astype(np.int64), S)


def test_table_builder_rejects_bad_arguments():
    lib = pa.load_library()
    buf = np.zeros(64, dtype=np.float32)
    assert lib.prefill_attn_rope_table_f32(0, 64, 1e4, buf.ctypes.data) == pa.PA_EINVAL
    assert lib.prefill_attn_rope_table_f32(1, 63, 1e4, buf.ctypes.data) == pa.PA_EINVAL
    assert lib.prefill_attn_rope_table_f32(1, 64, -1.0, buf.ctypes.data) == pa.PA_EINVAL
    assert lib.prefill_attn_rope_table_f32(1, 64, math.nan, buf.ctypes.data) == pa.PA_EINVAL
    assert lib.prefill_attn_rope_table_q14(1, 64, 1e4, None) == pa.PA_EINVAL


@pytest.mark.parametrize("args", [
    (0, 1, 128, 512, 1e4),      # no heads
    (32, 0, 128, 512, 1e4),     # no kv heads
    (32, 5, 128, 512, 1e4),     # kv heads do not divide heads
    (32, 32, 80, 512, 1e4),     # unsupported head_dim
    (32, 32, 128, 0, 1e4),      # empty table
    (32, 32, 128, (1 << 20) + 1, 1e4),
    (32, 32, 128, 512, 1.0),    # theta must exceed 1
    (32, 32, 128, 512, math.inf),
])
def test_init_rejects_bad_arguments(args):
    lib = pa.load_library()
    import ctypes
    h = ctypes.c_void_p(1234)
    assert lib.prefill_attn_init(ctypes.byref(h), *args) == pa.PA_EINVAL
    assert h.value is None
    assert lib.prefill_attn_init(None, 32, 32, 128, 512, 1e4) == pa.PA_EINVAL


def test_calls_on_null_handle():
    lib = pa.load_library()
    assert lib.prefill_attn_run(None, pa.PA_IN_BF16, 1, 16, 16, 16, 16, None, 16, 0.0, None) == pa.PA_EINVAL
    assert lib.prefill_attn_status(None, None) == pa.PA_EINVAL
    assert lib.prefill_attn_destroy(None) == pa.PA_OK
    assert lib.prefill_attn_debug_rope_i16(None, 1, 1, 16, 1, None, 16, None) == pa.PA_EINVAL
    assert lib.prefill_attn_debug_scores_i32(None, 1, 1, 16, 16, None, 16, None) == pa.PA_EINVAL
    assert lib.prefill_attn_kv_cache_update(None, pa.PA_IN_BF16, 1, 4, 16, 16, None, 16, 4, 16, 16, 8,
                                            None) == pa.PA_EINVAL
    assert lib.prefill_attn_run_cached(None, pa.PA_IN_BF16, 1, 4, 16, 16, 16, 8, 16, 4, None, 16, 0.0,
                                       None) == pa.PA_EINVAL
    assert lib.prefill_attn_decode(None, pa.PA_IN_BF16, 1, 16, 16, 16, 8, 16, 4, None, 16, 0.0, 0, None, 0,
                                   None) == pa.PA_EINVAL
    assert lib.prefill_attn_decode_workspace_size(None, 4, 8) == 0
    assert lib.prefill_attn_decode_noalloc(None, pa.PA_IN_BF16, 1, 16, 16, 16, 8, 16, 4, None, 16, 0.0, 0,
                                           None) == pa.PA_EINVAL
    assert lib.prefill_attn_decode_noalloc_scratch_bytes() == 8 << 20


@pytest.mark.parametrize("n_slots,start,count", [(128, 120, 12), (8, 0, 8), (5, 4, 23), (1, 0, 3), (16, 3, 0)])
def test_ring_map_matches_oracle(n_slots, start, count):
    got = pa.prefill_attn_ring_map(n_slots, start, count)
    assert got.dtype == np.int32
    assert got.astype(np.int64).tolist() == oracle.ring_index_map(n_slots, start, count).tolist()


@pytest.mark.parametrize("table,block,count", [([3, 0, 2], 4, 10), ([7], 16, 16), ([5, 1, 9, 2], 1, 4),
                                               ([2, 0], 64, 100)])
def test_paged_map_matches_oracle(table, block, count):
    got = pa.prefill_attn_paged_map(table, block, count)
    assert got.astype(np.int64).tolist() == oracle.paged_index_map(table, block, count).tolist()


def test_map_builders_reject_bad_arguments():
    lib = pa.load_library()
    buf = np.zeros(16, dtype=np.int32)
    bt = np.array([1, 2], dtype=np.int32)
    assert lib.prefill_attn_ring_map(0, 0, 4, buf.ctypes.data) == pa.PA_EINVAL        # no slots
    assert lib.prefill_attn_ring_map(8, 8, 4, buf.ctypes.data) == pa.PA_EINVAL        # start outside the ring
    assert lib.prefill_attn_ring_map(8, 0, -1, buf.ctypes.data) == pa.PA_EINVAL
    assert lib.prefill_attn_ring_map(8, 0, 4, None) == pa.PA_EINVAL
    assert lib.prefill_attn_paged_map(bt.ctypes.data, 2, 4, 9, buf.ctypes.data) == pa.PA_EINVAL  # 3 blocks needed
    assert lib.prefill_attn_paged_map(bt.ctypes.data, 2, 0, 4, buf.ctypes.data) == pa.PA_EINVAL  # block size 0
    neg = np.array([-1], dtype=np.int32)
    assert lib.prefill_attn_paged_map(neg.ctypes.data, 1, 4, 4, buf.ctypes.data) == pa.PA_EINVAL
    big = np.array([1 << 30], dtype=np.int32)
    assert lib.prefill_attn_paged_map(big.ctypes.data, 1, 4, 4, buf.ctypes.data) == pa.PA_EINVAL  # slot >= 2^31
    assert lib.prefill_attn_paged_map(None, 0, 4, 0, None) == pa.PA_OK


def test_strerror_covers_every_code():
    texts = {c: pa.prefill_attn_strerror(c) for c in (0, -1, -2, -3, -4, -5, -6, -7)}
    assert len(set(texts.values())) == 8
    assert pa.prefill_attn_strerror(-99) == "unknown status code"


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_init_without_device_reports_edevice():
    lib = pa.load_library()
    import ctypes
    h = ctypes.c_void_p()
    assert lib.prefill_attn_init(ctypes.byref(h), 32, 32, 128, 512, 1e4) == pa.PA_EDEVICE
    assert h.value is None
