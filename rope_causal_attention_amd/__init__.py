"""Python binding of libprefill_attn.so: fused RoPE causal prefill attention.

Argument marshalling only: every step of the attention runs in the HIP kernels
of the C-ABI library (``include/prefill_attn.h``).  PyTorch supplies device
memory and the stream.  There is no other implementation behind these names:
if the library is missing or cannot be loaded, every call raises.

torch is imported before the library is loaded so that the library's
``libamdhip64.so.7`` dependency resolves to the HIP runtime torch already has
in the process (one runtime, so torch's streams and pointers are valid in the
library); :func:`load_library` checks that only one HIP runtime is mapped.
"""

import ctypes
import os

import numpy as np
import torch

__all__ = [
    "PA_IN_F32", "PA_IN_BF16", "PA_IN_I16", "PA_IN_BF16_Q16", "PA_IN_I16_PWL",
    "PA_OK", "PA_EINVAL", "PA_ENOMEM", "PA_EDEVICE", "PA_ELAUNCH", "PA_ERANGE", "PA_ETOOBIG",
    "PA_EOVERFLOW",
    "PrefillAttnError", "load_library", "library_path",
    "prefill_attn_init", "prefill_attn_run", "prefill_attn_status", "prefill_attn_destroy",
    "prefill_attn_strerror", "prefill_attn_rope_table_f32", "prefill_attn_rope_table_q14",
    "prefill_attn_debug_rope_i16", "prefill_attn_debug_scores_i32", "prefill_attn_debug_scores_q16",
    "prefill_attn_kv_cache_update", "prefill_attn_run_cached", "prefill_attn_ring_map", "prefill_attn_paged_map",
    "prefill_attn_decode", "prefill_attn_decode_workspace_size",
    "prefill_attn_decode_noalloc", "prefill_attn_decode_noalloc_scratch_bytes", "prefill_attn_device_peak",
    "prefill_attn_run_cached_splitk", "prefill_attn_run_cached_workspace_size", "prefill_attn_run_cached_update",
    "PrefillAttention", "EXPORTED_SYMBOLS",
]

PA_IN_F32, PA_IN_BF16, PA_IN_I16, PA_IN_BF16_Q16, PA_IN_I16_PWL = 0, 1, 2, 3, 4
PA_OK, PA_EINVAL, PA_ENOMEM, PA_EDEVICE, PA_ELAUNCH, PA_ERANGE, PA_ETOOBIG, PA_EOVERFLOW = \
    0, -1, -2, -3, -4, -5, -6, -7

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libprefill_attn.so")

_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGNATURES = {
    "prefill_attn_init": (_I, [ctypes.POINTER(_P), _I, _I, _I, _I, ctypes.c_double]),
    "prefill_attn_run": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _P, ctypes.c_float, _P]),
    "prefill_attn_status": (_I, [_P, _P]),
    "prefill_attn_destroy": (_I, [_P]),
    "prefill_attn_strerror": (ctypes.c_char_p, [_I]),
    "prefill_attn_rope_table_f32": (_I, [_I, _I, ctypes.c_double, _P]),
    "prefill_attn_rope_table_q14": (_I, [_I, _I, ctypes.c_double, _P]),
    "prefill_attn_debug_rope_i16": (_I, [_P, _I, _I, _P, _I, _P, _P, _P]),
    "prefill_attn_debug_scores_i32": (_I, [_P, _I, _I, _P, _P, _P, _P, _P]),
    "prefill_attn_debug_scores_q16": (_I, [_P, _I, _I, _P, _P, _P, _P, _P]),
    "prefill_attn_kv_cache_update": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _I, _P]),
    "prefill_attn_run_cached": (_I, [_P, _I, _I, _I, _P, _P, _P, _I, _P, _I, _P, _P, ctypes.c_float, _P]),
    "prefill_attn_ring_map": (_I, [_I, _I, _I, _P]),
    "prefill_attn_paged_map": (_I, [_P, _I, _I, _I, _P]),
    "prefill_attn_decode_workspace_size": (ctypes.c_size_t, [_P, _I, _I]),
    "prefill_attn_run_cached_workspace_size": (ctypes.c_size_t, [_P, _I, _I, _I]),
    "prefill_attn_run_cached_splitk": (_I, [_P, _I, _I, _I, _P, _P, _P, _I, _P, _I, _P, _P, ctypes.c_float, _I,
                                            _P, ctypes.c_size_t, _P]),
    "prefill_attn_decode": (_I, [_P, _I, _I, _P, _P, _P, _I, _P, _I, _P, _P, ctypes.c_float, _I, _P,
                                 ctypes.c_size_t, _P]),
    "prefill_attn_run_cached_update": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _I, _P, _P, ctypes.c_float,
                                            _I, _P, ctypes.c_size_t, _P]),
    "prefill_attn_decode_noalloc": (_I, [_P, _I, _I, _P, _P, _P, _I, _P, _I, _P, _P, ctypes.c_float, _I, _P]),
    "prefill_attn_decode_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "prefill_attn_device_peak": (_I, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), _P]),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)

_lib = None


class PrefillAttnError(RuntimeError):
    def __init__(self, code, what):
        self.code = code
        super().__init__(f"{what}: {_strerror(code)} ({code})")


def library_path():
    return _LIB_PATH


def _hip_runtimes_mapped():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def load_library():
    """Load (once) and return the ctypes handle of libprefill_attn.so."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m rope_causal_attention_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"more than one HIP runtime is mapped into the process: {sorted(runtimes)}")
    _lib = lib
    return lib


def _strerror(code):
    try:
        return load_library().prefill_attn_strerror(int(code)).decode()
    except Exception:  # noqa: BLE001 - only used while formatting an error
        return "unknown status code"


def _check(code, what):
    if code != PA_OK:
        raise PrefillAttnError(code, what)


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


# ------------------------------------------------------------------ C calls

def prefill_attn_init(n_heads, n_kv_heads, head_dim, max_seq, rope_theta):
    """Create a handle on the current device (see prefill_attn_init in the header)."""
    h = _P()
    _check(load_library().prefill_attn_init(ctypes.byref(h), n_heads, n_kv_heads, head_dim, max_seq,
                                            float(rope_theta)), "prefill_attn_init")
    return h.value


def prefill_attn_run(handle, in_dtype, batch, seq_len, q, k, v, pos_offsets, out, score_scale=0.0,
                     stream=None):
    """Enqueue one fused attention pass; tensors or raw device pointers."""
    _check(load_library().prefill_attn_run(handle, in_dtype, batch, seq_len, _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(pos_offsets), _ptr(out), float(score_scale), _stream(stream)),
           "prefill_attn_run")


def prefill_attn_status(handle, stream=None):
    """Synchronise the stream; return PA_OK, PA_ERANGE or PA_EOVERFLOW (and clear the flags)."""
    code = load_library().prefill_attn_status(handle, _stream(stream))
    if code not in (PA_OK, PA_ERANGE, PA_EOVERFLOW):
        raise PrefillAttnError(code, "prefill_attn_status")
    return code


def prefill_attn_destroy(handle):
    _check(load_library().prefill_attn_destroy(handle), "prefill_attn_destroy")


def prefill_attn_strerror(code):
    return _strerror(code)


def prefill_attn_rope_table_f32(max_seq, head_dim, rope_theta):
    """Host table [max_seq][head_dim/2][2] float32 (cos, sin)."""
    out = np.empty((max_seq, head_dim // 2, 2), dtype=np.float32)
    _check(load_library().prefill_attn_rope_table_f32(max_seq, head_dim, float(rope_theta),
                                                      out.ctypes.data), "prefill_attn_rope_table_f32")
    return out


def prefill_attn_rope_table_q14(max_seq, head_dim, rope_theta):
    """Host table [max_seq][head_dim/2][2] int16 (C, S) in Q1.14."""
    out = np.empty((max_seq, head_dim // 2, 2), dtype=np.int16)
    _check(load_library().prefill_attn_rope_table_q14(max_seq, head_dim, float(rope_theta),
                                                      out.ctypes.data), "prefill_attn_rope_table_q14")
    return out


def prefill_attn_debug_rope_i16(handle, batch, seq_len, x, n_heads_x, pos_offsets, x_rot, stream=None):
    _check(load_library().prefill_attn_debug_rope_i16(handle, batch, seq_len, _ptr(x), n_heads_x,
                                                      _ptr(pos_offsets), _ptr(x_rot), _stream(stream)),
           "prefill_attn_debug_rope_i16")


def prefill_attn_debug_scores_i32(handle, batch, seq_len, q, k, pos_offsets, scores, stream=None):
    _check(load_library().prefill_attn_debug_scores_i32(handle, batch, seq_len, _ptr(q), _ptr(k),
                                                        _ptr(pos_offsets), _ptr(scores), _stream(stream)),
           "prefill_attn_debug_scores_i32")


def prefill_attn_debug_scores_q16(handle, batch, seq_len, q, k, pos_offsets, scores, stream=None):
    _check(load_library().prefill_attn_debug_scores_q16(handle, batch, seq_len, _ptr(q), _ptr(k),
                                                        _ptr(pos_offsets), _ptr(scores), _stream(stream)),
           "prefill_attn_debug_scores_q16")


def prefill_attn_kv_cache_update(handle, in_dtype, batch, seq_len, k_new, v_new, pos_offsets, kv_map, map_stride,
                                 k_cache, v_cache, n_slots, stream=None):
    """Copy the new tokens' K/V into their cache slots (see the header)."""
    _check(load_library().prefill_attn_kv_cache_update(handle, in_dtype, batch, seq_len, _ptr(k_new), _ptr(v_new),
                                                       _ptr(pos_offsets), _ptr(kv_map), map_stride, _ptr(k_cache),
                                                       _ptr(v_cache), n_slots, _stream(stream)),
           "prefill_attn_kv_cache_update")


def prefill_attn_run_cached(handle, in_dtype, batch, seq_len, q, k_cache, v_cache, n_slots, kv_map, map_stride,
                            pos_offsets, out, score_scale=0.0, stream=None):
    """Enqueue one cached (chunked) prefill pass (see the header)."""
    _check(load_library().prefill_attn_run_cached(handle, in_dtype, batch, seq_len, _ptr(q), _ptr(k_cache),
                                                  _ptr(v_cache), n_slots, _ptr(kv_map), map_stride,
                                                  _ptr(pos_offsets), _ptr(out), float(score_scale),
                                                  _stream(stream)),
           "prefill_attn_run_cached")


def prefill_attn_ring_map(n_slots, start, count):
    """Host int32 map[j] = (start + j) mod n_slots, j < count."""
    out = np.empty(max(count, 1), dtype=np.int32)
    _check(load_library().prefill_attn_ring_map(n_slots, start, count, out.ctypes.data), "prefill_attn_ring_map")
    return out[:count]


def prefill_attn_paged_map(block_table, block_size, count):
    """Host int32 map[j] = block_table[j // block_size] * block_size + j % block_size."""
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    out = np.empty(max(count, 1), dtype=np.int32)
    _check(load_library().prefill_attn_paged_map(bt.ctypes.data if bt.size else None, bt.size, block_size, count,
                                                 out.ctypes.data), "prefill_attn_paged_map")
    return out[:count]


def prefill_attn_run_cached_workspace_size(handle, batch, seq_len, n_split):
    """Bytes of workspace a split-K cached run with n_split > 1 needs (0 for n_split = 1)."""
    return int(load_library().prefill_attn_run_cached_workspace_size(handle, batch, seq_len, n_split))


def prefill_attn_run_cached_splitk(handle, in_dtype, batch, seq_len, q, k_cache, v_cache, n_slots, kv_map,
                                   map_stride, pos_offsets, out, score_scale=0.0, n_split=0, workspace=None,
                                   workspace_bytes=0, stream=None):
    """Enqueue a split-K cached prefill pass (see the header)."""
    _check(load_library().prefill_attn_run_cached_splitk(handle, in_dtype, batch, seq_len, _ptr(q), _ptr(k_cache),
                                                         _ptr(v_cache), n_slots, _ptr(kv_map), map_stride,
                                                         _ptr(pos_offsets), _ptr(out), float(score_scale), n_split,
                                                         _ptr(workspace), int(workspace_bytes), _stream(stream)),
           "prefill_attn_run_cached_splitk")


def prefill_attn_run_cached_update(handle, in_dtype, batch, seq_len, q, k_new, v_new, k_cache, v_cache, n_slots,
                                   kv_map, map_stride, pos_offsets, out, score_scale=0.0, n_split=1, workspace=None,
                                   workspace_bytes=0, stream=None):
    """Enqueue the cache update of a chunk and its cached prefill in one launch (see the header)."""
    _check(load_library().prefill_attn_run_cached_update(handle, in_dtype, batch, seq_len, _ptr(q), _ptr(k_new),
                                                         _ptr(v_new), _ptr(k_cache), _ptr(v_cache), n_slots,
                                                         _ptr(kv_map), map_stride, _ptr(pos_offsets), _ptr(out),
                                                         float(score_scale), n_split, _ptr(workspace),
                                                         int(workspace_bytes), _stream(stream)),
           "prefill_attn_run_cached_update")


def prefill_attn_decode_workspace_size(handle, batch, n_split):
    """Bytes of workspace a decode call with n_split > 1 needs (0 for n_split = 1)."""
    return int(load_library().prefill_attn_decode_workspace_size(handle, batch, n_split))


def prefill_attn_decode(handle, in_dtype, batch, q, k_cache, v_cache, n_slots, kv_map, map_stride, pos_offsets,
                        out, score_scale=0.0, n_split=0, workspace=None, workspace_bytes=0, stream=None):
    """Enqueue one decode-attention pass (see the header)."""
    _check(load_library().prefill_attn_decode(handle, in_dtype, batch, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                              n_slots, _ptr(kv_map), map_stride, _ptr(pos_offsets), _ptr(out),
                                              float(score_scale), n_split, _ptr(workspace), int(workspace_bytes),
                                              _stream(stream)),
           "prefill_attn_decode")


def prefill_attn_decode_noalloc(handle, in_dtype, batch, q, k_cache, v_cache, n_slots, kv_map, map_stride,
                                pos_offsets, out, score_scale=0.0, n_split=0, stream=None):
    """Enqueue one decode pass with the partials in the library's fixed scratch (see the header)."""
    _check(load_library().prefill_attn_decode_noalloc(handle, in_dtype, batch, _ptr(q), _ptr(k_cache),
                                                      _ptr(v_cache), n_slots, _ptr(kv_map), map_stride,
                                                      _ptr(pos_offsets), _ptr(out), float(score_scale), n_split,
                                                      _stream(stream)),
           "prefill_attn_decode_noalloc")


def prefill_attn_decode_noalloc_scratch_bytes():
    """Bytes of the fixed scratch that prefill_attn_decode_noalloc's partials use."""
    return int(load_library().prefill_attn_decode_noalloc_scratch_bytes())


def prefill_attn_device_peak(stream=None):
    """(measured matrix-core TFLOP/s, shader clock GHz) of the current device."""
    tf, ghz = ctypes.c_double(), ctypes.c_double()
    _check(load_library().prefill_attn_device_peak(ctypes.byref(tf), ctypes.byref(ghz), _stream(stream)),
           "prefill_attn_device_peak")
    return tf.value, ghz.value


# ------------------------------------------------------------- tensor helper

_DTYPES = {torch.float32: PA_IN_F32, torch.bfloat16: PA_IN_BF16, torch.int16: PA_IN_I16}


class PrefillAttention:
    """A handle plus tensor marshalling: ``attn(q, k, v) -> O`` (float32).

    q [B][S][Hq][D], k/v [B][S][Hkv][D] on the handle's device, contiguous;
    float32 or bfloat16 Q/K/V, or int16 Q/K with bfloat16 V.
    """

    def __init__(self, n_heads, n_kv_heads, head_dim, max_seq, rope_theta=10000.0):
        self.n_heads, self.n_kv_heads, self.head_dim = n_heads, n_kv_heads, head_dim
        self.max_seq, self.rope_theta = max_seq, rope_theta
        self.handle = prefill_attn_init(n_heads, n_kv_heads, head_dim, max_seq, rope_theta)

    def close(self):
        if self.handle:
            prefill_attn_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass

    @staticmethod
    def _dtype(q, quantize):
        if q.dtype not in _DTYPES:
            raise TypeError(f"unsupported q dtype {q.dtype}")
        if quantize:
            if q.dtype != torch.bfloat16:
                raise TypeError("quantize=True takes bfloat16 q/k/v")
            return PA_IN_BF16_Q16
        return _DTYPES[q.dtype]

    def _validate(self, q, k, v, pos_offsets, out, quantize=False):
        dt = self._dtype(q, quantize)
        want_kv = q.dtype
        if k.dtype != want_kv or v.dtype != (torch.bfloat16 if dt == PA_IN_I16 else want_kv):
            raise TypeError("k must match q's dtype; v must too (bfloat16 for int16 q/k)")
        B, S, Hq, D = q.shape
        if Hq != self.n_heads or D != self.head_dim:
            raise ValueError("q shape does not match the handle")
        if tuple(k.shape) != (B, S, self.n_kv_heads, D) or tuple(v.shape) != (B, S, self.n_kv_heads, D):
            raise ValueError("k/v shape must be [B][S][n_kv_heads][head_dim]")
        for t in (q, k, v) + ((out,) if out is not None else ()):
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError("tensors must be contiguous device tensors")
        if out is not None and (out.dtype != torch.float32 or tuple(out.shape) != (B, S, Hq, D)):
            raise ValueError("out must be float32 [B][S][n_heads][head_dim]")
        if pos_offsets is not None and (pos_offsets.dtype != torch.int32 or pos_offsets.numel() != B
                                        or not pos_offsets.is_cuda):
            raise ValueError("pos_offsets must be a device int32 tensor with one entry per batch element")
        return dt, B, S

    def __call__(self, q, k, v, pos_offsets=None, score_scale=0.0, out=None, stream=None, quantize=False,
                 pwl_softmax=False):
        """O (float32) of q [B][S][Hq][D], k/v [B][S][Hkv][D].  quantize=True runs bfloat16
        inputs through the in-kernel per-token int16 quantisation (PA_IN_BF16_Q16);
        pwl_softmax=True runs int16 inputs with the piecewise-linear softmax (PA_IN_I16_PWL)."""
        dt, B, S = self._validate(q, k, v, pos_offsets, out, quantize)
        if pwl_softmax:
            if dt != PA_IN_I16:
                raise TypeError("pwl_softmax=True takes int16 q/k")
            dt = PA_IN_I16_PWL
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        prefill_attn_run(self.handle, dt, B, S, q, k, v, pos_offsets, out, score_scale, stream)
        return out

    def status(self, stream=None):
        return prefill_attn_status(self.handle, stream)

    # ---- KV cache (chunked prefill)

    def _check_cache(self, k_cache, v_cache, kv_map, dt, B):
        if k_cache.dim() != 3 or tuple(k_cache.shape[1:]) != (self.n_kv_heads, self.head_dim):
            raise ValueError("caches must be [n_slots][n_kv_heads][head_dim]")
        if tuple(v_cache.shape) != tuple(k_cache.shape):
            raise ValueError("k_cache and v_cache must have the same shape")
        if k_cache.dtype != {PA_IN_F32: torch.float32, PA_IN_BF16: torch.bfloat16, PA_IN_I16: torch.int16,
                             PA_IN_BF16_Q16: torch.bfloat16}[dt] or \
                v_cache.dtype != (torch.bfloat16 if dt == PA_IN_I16 else k_cache.dtype):
            raise TypeError("cache dtypes must match the inputs (int16 K with bfloat16 V for the int16 variant)")
        if kv_map.dtype != torch.int32 or kv_map.dim() != 2 or kv_map.shape[0] != B:
            raise ValueError("kv_map must be int32 [batch][map_stride]")
        for t in (k_cache, v_cache, kv_map):
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError("caches and kv_map must be contiguous device tensors")
        return k_cache.shape[0], kv_map.shape[1]

    def kv_cache_update(self, k_new, v_new, k_cache, v_cache, kv_map, pos_offsets=None, stream=None):
        """Write k_new/v_new [B][S][Hkv][D] to slots kv_map[b][pos_offsets[b] + i]."""
        dt = _DTYPES.get(k_new.dtype)
        if dt is None:
            raise TypeError(f"unsupported dtype {k_new.dtype}")
        B, S = k_new.shape[:2]
        if tuple(k_new.shape) != (B, S, self.n_kv_heads, self.head_dim) or v_new.shape != k_new.shape:
            raise ValueError("k_new/v_new must be [B][S][n_kv_heads][head_dim]")
        if not (k_new.is_contiguous() and v_new.is_contiguous()):
            raise ValueError("k_new/v_new must be contiguous")
        n_slots, stride = self._check_cache(k_cache, v_cache, kv_map, dt, B)
        prefill_attn_kv_cache_update(self.handle, dt, B, S, k_new, v_new, pos_offsets, kv_map, stride, k_cache,
                                     v_cache, n_slots, stream)

    def run_cached(self, q, k_cache, v_cache, kv_map, pos_offsets=None, score_scale=0.0, out=None, stream=None,
                   quantize=False, n_split=1, workspace=None):
        """Chunked prefill: queries q [B][S][Hq][D] at positions pos_offsets[b] + i
        against the cached logical keys 0 .. pos_offsets[b] + i.  Returns O (float32).
        n_split != 1 (0 = chosen by the library) with a device workspace tensor splits
        the keys over several workgroups (prefill_attn_run_cached_splitk)."""
        dt = self._dtype(q, quantize)
        B, S, Hq, D = q.shape
        if Hq != self.n_heads or D != self.head_dim or not q.is_cuda or not q.is_contiguous():
            raise ValueError("q must be a contiguous device tensor [B][S][n_heads][head_dim]")
        n_slots, stride = self._check_cache(k_cache, v_cache, kv_map, dt, B)
        if pos_offsets is not None and (pos_offsets.dtype != torch.int32 or pos_offsets.numel() != B
                                        or not pos_offsets.is_cuda):
            raise ValueError("pos_offsets must be a device int32 tensor with one entry per batch element")
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        elif out.dtype != torch.float32 or tuple(out.shape) != tuple(q.shape) or not out.is_contiguous():
            raise ValueError("out must be contiguous float32 [B][S][n_heads][head_dim]")
        if workspace is None and n_split == 1:
            prefill_attn_run_cached(self.handle, dt, B, S, q, k_cache, v_cache, n_slots, kv_map, stride,
                                    pos_offsets, out, score_scale, stream)
        else:
            ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
            prefill_attn_run_cached_splitk(self.handle, dt, B, S, q, k_cache, v_cache, n_slots, kv_map, stride,
                                           pos_offsets, out, score_scale, n_split, workspace, ws_bytes, stream)
        return out

    def run_cached_update(self, q, k_new, v_new, k_cache, v_cache, kv_map, pos_offsets=None, score_scale=0.0,
                          out=None, stream=None, quantize=False, n_split=1, workspace=None):
        """kv_cache_update of the chunk's k_new/v_new followed by run_cached, as one
        launch (prefill_attn_run_cached_update).  Returns O (float32)."""
        dt = self._dtype(q, quantize)
        B, S, Hq, D = q.shape
        if Hq != self.n_heads or D != self.head_dim or not q.is_cuda or not q.is_contiguous():
            raise ValueError("q must be a contiguous device tensor [B][S][n_heads][head_dim]")
        if tuple(k_new.shape) != (B, S, self.n_kv_heads, self.head_dim) or v_new.shape != k_new.shape:
            raise ValueError("k_new/v_new must be [B][S][n_kv_heads][head_dim]")
        if not (k_new.is_contiguous() and v_new.is_contiguous()):
            raise ValueError("k_new/v_new must be contiguous")
        n_slots, stride = self._check_cache(k_cache, v_cache, kv_map, dt, B)
        if pos_offsets is not None and (pos_offsets.dtype != torch.int32 or pos_offsets.numel() != B
                                        or not pos_offsets.is_cuda):
            raise ValueError("pos_offsets must be a device int32 tensor with one entry per batch element")
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        elif out.dtype != torch.float32 or tuple(out.shape) != tuple(q.shape) or not out.is_contiguous():
            raise ValueError("out must be contiguous float32 [B][S][n_heads][head_dim]")
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        prefill_attn_run_cached_update(self.handle, dt, B, S, q, k_new, v_new, k_cache, v_cache, n_slots, kv_map,
                                       stride, pos_offsets, out, score_scale, n_split, workspace, ws_bytes, stream)
        return out

    def decode(self, q, k_cache, v_cache, kv_map, pos_offsets=None, score_scale=0.0, n_split=0, workspace=None,
               out=None, stream=None):
        """One new token per sequence: q [B][n_heads][head_dim] (float32 or bfloat16) at
        position pos_offsets[b] against cached keys 0 .. pos_offsets[b].  Returns O
        float32 [B][n_heads][head_dim].  workspace: a device tensor (any dtype) or None."""
        if q.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("decode takes float32 or bfloat16 q")
        dt = _DTYPES[q.dtype]
        B = q.shape[0]
        if tuple(q.shape) != (B, self.n_heads, self.head_dim) or not q.is_cuda or not q.is_contiguous():
            raise ValueError("q must be a contiguous device tensor [B][n_heads][head_dim]")
        n_slots, stride = self._check_cache(k_cache, v_cache, kv_map, dt, B)
        if pos_offsets is not None and (pos_offsets.dtype != torch.int32 or pos_offsets.numel() != B
                                        or not pos_offsets.is_cuda):
            raise ValueError("pos_offsets must be a device int32 tensor with one entry per batch element")
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        elif out.dtype != torch.float32 or tuple(out.shape) != tuple(q.shape) or not out.is_contiguous():
            raise ValueError("out must be contiguous float32 [B][n_heads][head_dim]")
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        prefill_attn_decode(self.handle, dt, B, q, k_cache, v_cache, n_slots, kv_map, stride, pos_offsets, out,
                            score_scale, n_split, workspace, ws_bytes, stream)
        return out
