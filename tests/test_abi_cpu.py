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


def test_strerror_covers_every_code():
    texts = {c: pa.prefill_attn_strerror(c) for c in (0, -1, -2, -3, -4, -5)}
    assert len(set(texts.values())) == 6
    assert pa.prefill_attn_strerror(-99) == "unknown status code"


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_init_without_device_reports_edevice():
    lib = pa.load_library()
    import ctypes
    h = ctypes.c_void_p()
    assert lib.prefill_attn_init(ctypes.byref(h), 32, 32, 128, 512, 1e4) == pa.PA_EDEVICE
    assert h.value is None
