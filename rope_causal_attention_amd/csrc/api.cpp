// C-ABI of the fused RoPE causal prefill attention library.
//
// The three-call shape (init binds the constant data and reserves memory once,
// run computes, cleanup releases) follows the interface of the 2kiu.com
// retelling of the hand-written prefill engine (§1.2); the "no allocation after
// start-up" rule is the page titled "手写内核实现6倍prefill加速" (§2.2).  Unlike
// those pages' interface this one reports every failure as a status code.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <algorithm>
#include <new>
#include <vector>

#include "internal.h"
#include "prefill_attn.h"

struct prefill_attn {
    int device;
    int n_heads;
    int n_kv_heads;
    int head_dim;
    int max_seq;
    double rope_theta;
    float* d_rope_f32;
    int16_t* d_rope_q14;
    int* d_status;
};

namespace {

constexpr int kMaxSeq = 1 << 20;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

void free_handle(prefill_attn* h) {
    if (!h) return;
    if (h->d_rope_f32) (void)hipFree(h->d_rope_f32);
    if (h->d_rope_q14) (void)hipFree(h->d_rope_q14);
    if (h->d_status) (void)hipFree(h->d_status);
    delete h;
}

// Checks shared by run and the test exports; fills the common launch arguments.
int prepare(const prefill_attn* h, int batch, int seq_len, const int32_t* pos_offsets, pa::RunArgs& a) {
    if (!h || batch < 0 || seq_len < 0 || seq_len > h->max_seq) return PA_EINVAL;
    if (pos_offsets && !aligned4(pos_offsets)) return PA_EINVAL;
    // every index the kernels form stays below 2^62; the grid below 2^31 workgroups
    const long long qblocks = (static_cast<long long>(seq_len) + 127) / 128;
    if (qblocks * batch * h->n_heads > 0x7fffffffLL) return PA_EINVAL;
    std::memset(&a, 0, sizeof(a));
    a.pos_offsets = pos_offsets;
    a.rope_f32 = h->d_rope_f32;
    a.rope_q14 = h->d_rope_q14;
    a.status = h->d_status;
    a.batch = batch;
    a.seq_len = seq_len;
    a.n_heads = h->n_heads;
    a.n_kv_heads = h->n_kv_heads;
    a.max_seq = h->max_seq;
    return PA_OK;
}

}  // namespace

extern "C" int prefill_attn_init(prefill_attn** out, int n_heads, int n_kv_heads, int head_dim, int max_seq,
                                 double rope_theta) {
    if (!out) return PA_EINVAL;
    *out = nullptr;
    if (n_heads < 1 || n_kv_heads < 1 || n_heads % n_kv_heads != 0) return PA_EINVAL;
    if (head_dim != 64 && head_dim != 96 && head_dim != 128) return PA_EINVAL;
    if (max_seq < 1 || max_seq > kMaxSeq) return PA_EINVAL;
    if (!std::isfinite(rope_theta) || rope_theta <= 1.0) return PA_EINVAL;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PA_EDEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return PA_EDEVICE;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return PA_EDEVICE;

    const size_t n = static_cast<size_t>(max_seq) * head_dim;  // (cos, sin) pairs x D/2 per row
    std::vector<float> t32;
    std::vector<int16_t> t14;
    try {
        t32.resize(n);
        t14.resize(n);
    } catch (const std::bad_alloc&) {
        return PA_ENOMEM;
    }
    if (pa::build_rope_tables(max_seq, head_dim, rope_theta, t32.data(), t14.data()) != PA_OK)
        return PA_EINVAL;

    prefill_attn* h = new (std::nothrow) prefill_attn{dev, n_heads, n_kv_heads, head_dim, max_seq, rope_theta,
                                                      nullptr, nullptr, nullptr};
    if (!h) return PA_ENOMEM;
    if (hipMalloc(&h->d_rope_f32, n * sizeof(float)) != hipSuccess ||
        hipMalloc(&h->d_rope_q14, n * sizeof(int16_t)) != hipSuccess ||
        hipMalloc(&h->d_status, sizeof(int)) != hipSuccess) {
        free_handle(h);
        return PA_ENOMEM;
    }
    if (hipMemcpy(h->d_rope_f32, t32.data(), n * sizeof(float), hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(h->d_rope_q14, t14.data(), n * sizeof(int16_t), hipMemcpyHostToDevice) != hipSuccess ||
        hipMemset(h->d_status, 0, sizeof(int)) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        free_handle(h);
        return PA_ELAUNCH;
    }
    // The no-allocation decode's scratch address on this device (looked up once).
    float* scratch = nullptr;
    if (pa::noalloc_scratch(&scratch) != hipSuccess) {
        free_handle(h);
        return PA_ELAUNCH;
    }
    *out = h;
    return PA_OK;
}

extern "C" int prefill_attn_run(const prefill_attn* h, int in_dtype, int batch, int seq_len, const void* q,
                                const void* k, const void* v, const int32_t* pos_offsets, float* out,
                                float score_scale, void* stream) {
    pa::RunArgs a;
    const int rc = prepare(h, batch, seq_len, pos_offsets, a);
    if (rc != PA_OK) return rc;
    if (in_dtype != PA_IN_F32 && in_dtype != PA_IN_BF16 && in_dtype != PA_IN_I16 && in_dtype != PA_IN_BF16_Q16 &&
        in_dtype != PA_IN_I16_PWL)
        return PA_EINVAL;
    if (!std::isfinite(score_scale)) return PA_EINVAL;
    if (batch == 0 || seq_len == 0) return PA_OK;
    if (!q || !k || !v || !out || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return PA_EINVAL;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.score_scale = score_scale != 0.0f ? score_scale : 1.0f / std::sqrt(static_cast<float>(h->head_dim));
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (in_dtype) {
        case PA_IN_F32: e = pa::launch_attn_f32(h->head_dim, a, s); break;
        case PA_IN_BF16: e = pa::launch_attn_bf16(h->head_dim, a, s); break;
        case PA_IN_BF16_Q16: e = pa::launch_attn_i16q(h->head_dim, a, s); break;
        case PA_IN_I16_PWL: e = pa::launch_attn_i16pwl(h->head_dim, a, s); break;
        default: e = pa::launch_attn_i16(h->head_dim, a, s); break;
    }
    return e == hipSuccess ? PA_OK : PA_ELAUNCH;
}

namespace {

int elem_bytes(int in_dtype) {
    switch (in_dtype) {
        case PA_IN_F32: return 4;
        case PA_IN_BF16: return 2;
        case PA_IN_I16: return 2;  // int16 K, bf16 V
        case PA_IN_BF16_Q16: return 2;
        default: return 0;
    }
}

// Cache-shape checks shared by the cache update and the cached run.
int check_cache(const prefill_attn* h, int el, int seq_len, int n_slots, const int32_t* kv_map, int map_stride,
                const void* k_cache, const void* v_cache) {
    if (el == 0 || n_slots < 1 || map_stride < 1 || map_stride < seq_len) return PA_EINVAL;
    // slot offsets are 32-bit byte offsets inside the kernels
    const unsigned long long bytes = static_cast<unsigned long long>(n_slots) * h->n_kv_heads * h->head_dim * el;
    if (bytes > 0xffffffffULL) return PA_EINVAL;
    if (!kv_map || !aligned4(kv_map)) return PA_EINVAL;
    if (!k_cache || !v_cache || !aligned16(k_cache) || !aligned16(v_cache)) return PA_EINVAL;
    return PA_OK;
}

}  // namespace

extern "C" int prefill_attn_kv_cache_update(const prefill_attn* h, int in_dtype, int batch, int seq_len,
                                            const void* k_new, const void* v_new, const int32_t* pos_offsets,
                                            const int32_t* kv_map, int map_stride, void* k_cache, void* v_cache,
                                            int n_slots, void* stream) {
    pa::RunArgs a;
    int rc = prepare(h, batch, seq_len, pos_offsets, a);
    if (rc != PA_OK) return rc;
    const int el = elem_bytes(in_dtype);
    if (el == 0) return PA_EINVAL;
    if (batch == 0 || seq_len == 0) return PA_OK;
    rc = check_cache(h, el, seq_len, n_slots, kv_map, map_stride, k_cache, v_cache);
    if (rc != PA_OK) return rc;
    if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return PA_EINVAL;
    a.k = k_new;
    a.v = v_new;
    a.kv_map = kv_map;
    a.map_stride = map_stride;
    a.n_slots = n_slots;
    hipError_t e = pa::launch_kv_cache_update(h->head_dim, el, a, k_cache, v_cache, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ELAUNCH;
}

namespace {

// run_cached, optionally with the chunk's own K/V (k_new, v_new: read by the
// attention for the chunk's keys and written to the cache by the same launch).
int run_cached_impl(const prefill_attn* h, int in_dtype, int batch, int seq_len, const void* q, const void* k_new,
                    const void* v_new, const void* k_cache, const void* v_cache, int n_slots, const int32_t* kv_map,
                    int map_stride, const int32_t* pos_offsets, float* out, float score_scale, void* stream) {
    pa::RunArgs a;
    int rc = prepare(h, batch, seq_len, pos_offsets, a);
    if (rc != PA_OK) return rc;
    const int el = elem_bytes(in_dtype);
    if (el == 0 || !std::isfinite(score_scale)) return PA_EINVAL;
    if (batch == 0 || seq_len == 0) return PA_OK;
    rc = check_cache(h, el, seq_len, n_slots, kv_map, map_stride, k_cache, v_cache);
    if (rc != PA_OK) return rc;
    if (!q || !out || !aligned16(q) || !aligned16(out)) return PA_EINVAL;
    if (k_new && (!aligned16(k_new) || !v_new || !aligned16(v_new))) return PA_EINVAL;
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.k_new = k_new;
    a.v_new = v_new;
    a.out = out;
    a.kv_map = kv_map;
    a.map_stride = map_stride;
    a.n_slots = n_slots;
    a.score_scale = score_scale != 0.0f ? score_scale : 1.0f / std::sqrt(static_cast<float>(h->head_dim));
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (in_dtype) {
        case PA_IN_F32: e = pa::launch_attn_f32(h->head_dim, a, s); break;
        case PA_IN_BF16: e = pa::launch_attn_bf16(h->head_dim, a, s); break;
        case PA_IN_BF16_Q16: e = pa::launch_attn_i16q(h->head_dim, a, s); break;
        default: e = pa::launch_attn_i16(h->head_dim, a, s); break;
    }
    return e == hipSuccess ? PA_OK : PA_ELAUNCH;
}

}  // namespace

extern "C" int prefill_attn_run_cached(const prefill_attn* h, int in_dtype, int batch, int seq_len, const void* q,
                                       const void* k_cache, const void* v_cache, int n_slots, const int32_t* kv_map,
                                       int map_stride, const int32_t* pos_offsets, float* out, float score_scale,
                                       void* stream) {
    return run_cached_impl(h, in_dtype, batch, seq_len, q, nullptr, nullptr, k_cache, v_cache, n_slots, kv_map,
                           map_stride, pos_offsets, out, score_scale, stream);
}

namespace {

size_t split_ws_bytes(const prefill_attn* h, int batch, int seq_len, int n_split) {
    return static_cast<size_t>(batch) * seq_len * h->n_heads * n_split * (h->head_dim + 2) * sizeof(float);
}

}  // namespace

extern "C" size_t prefill_attn_run_cached_workspace_size(const prefill_attn* h, int batch, int seq_len,
                                                         int n_split) {
    if (!h || batch < 0 || seq_len < 0 || n_split < 1) return 0;
    return n_split == 1 ? 0 : split_ws_bytes(h, batch, seq_len, n_split);
}

namespace {

int splitk_impl(const prefill_attn* h, int in_dtype, int batch, int seq_len, const void* q, const void* k_new,
                const void* v_new, const void* k_cache, const void* v_cache, int n_slots, const int32_t* kv_map,
                int map_stride, const int32_t* pos_offsets, float* out, float score_scale, int n_split,
                void* workspace, size_t workspace_bytes, void* stream) {
    if (!h || n_split < 0) return PA_EINVAL;
    if (workspace && !aligned16(workspace)) return PA_EINVAL;
    if (in_dtype == PA_IN_F32 || batch <= 0 || seq_len <= 0) n_split = 1;  // fp32 kernel has no split
    if (n_split == 0) {
        // Split only a grid that leaves CUs idle (under 256 eight-wave workgroups):
        // aim at one round of them (one per CU; a second round doubled the
        // partials to merge and measured slower), at least four 64-key tiles
        // per split.
        const long long wgs256 = static_cast<long long>((seq_len + 255) / 256) * batch * h->n_heads;
        n_split = wgs256 >= 256 ? 1 : static_cast<int>((256 + wgs256 - 1) / wgs256);
        n_split = std::min(n_split, std::max(1, map_stride / (4 * 64)));
    }
    if (n_split > 1 && (!workspace || workspace_bytes < split_ws_bytes(h, batch, seq_len, 2))) n_split = 1;
    while (n_split > 1 && split_ws_bytes(h, batch, seq_len, n_split) > workspace_bytes) --n_split;
    if (n_split == 1)
        return run_cached_impl(h, in_dtype, batch, seq_len, q, k_new, v_new, k_cache, v_cache, n_slots, kv_map,
                               map_stride, pos_offsets, out, score_scale, stream);

    pa::RunArgs a;
    int rc = prepare(h, batch, seq_len, pos_offsets, a);
    if (rc != PA_OK) return rc;
    const int el = elem_bytes(in_dtype);
    if (el == 0 || !std::isfinite(score_scale)) return PA_EINVAL;
    rc = check_cache(h, el, seq_len, n_slots, kv_map, map_stride, k_cache, v_cache);
    if (rc != PA_OK) return rc;
    if (!q || !out || !aligned16(q) || !aligned16(out)) return PA_EINVAL;
    if (k_new && (!aligned16(k_new) || !v_new || !aligned16(v_new))) return PA_EINVAL;
    const long long grid = ((static_cast<long long>(seq_len) + 127) / 128) * batch * h->n_heads * n_split;
    if (grid > 0x7fffffffLL) return PA_EINVAL;
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.k_new = k_new;
    a.v_new = v_new;
    a.out = out;
    a.kv_map = kv_map;
    a.map_stride = map_stride;
    a.n_slots = n_slots;
    a.n_split = n_split;
    a.ws = static_cast<float*>(workspace);
    a.score_scale = score_scale != 0.0f ? score_scale : 1.0f / std::sqrt(static_cast<float>(h->head_dim));
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (in_dtype) {
        case PA_IN_BF16: e = pa::launch_attn_bf16(h->head_dim, a, s); break;
        case PA_IN_BF16_Q16: e = pa::launch_attn_i16q(h->head_dim, a, s); break;
        default: e = pa::launch_attn_i16(h->head_dim, a, s); break;
    }
    if (e != hipSuccess) return PA_ELAUNCH;
    pa::DecodeArgs m;
    std::memset(&m, 0, sizeof(m));
    m.out = out;
    m.ws = a.ws;
    m.batch = batch * seq_len;
    m.n_heads = h->n_heads;
    m.n_split = n_split;
    e = pa::launch_split_merge(h->head_dim, m, s);
    return e == hipSuccess ? PA_OK : PA_ELAUNCH;
}

}  // namespace

extern "C" int prefill_attn_run_cached_splitk(const prefill_attn* h, int in_dtype, int batch, int seq_len,
                                              const void* q, const void* k_cache, const void* v_cache, int n_slots,
                                              const int32_t* kv_map, int map_stride, const int32_t* pos_offsets,
                                              float* out, float score_scale, int n_split, void* workspace,
                                              size_t workspace_bytes, void* stream) {
    return splitk_impl(h, in_dtype, batch, seq_len, q, nullptr, nullptr, k_cache, v_cache, n_slots, kv_map,
                       map_stride, pos_offsets, out, score_scale, n_split, workspace, workspace_bytes, stream);
}

extern "C" int prefill_attn_run_cached_update(const prefill_attn* h, int in_dtype, int batch, int seq_len,
                                              const void* q, const void* k_new, const void* v_new, void* k_cache,
                                              void* v_cache, int n_slots, const int32_t* kv_map, int map_stride,
                                              const int32_t* pos_offsets, float* out, float score_scale, int n_split,
                                              void* workspace, size_t workspace_bytes, void* stream) {
    if (!h) return PA_EINVAL;
    if (!k_new || !v_new) return PA_EINVAL;
    if (in_dtype == PA_IN_F32) {
        // the fp32 kernel reads every key from the cache: the update runs first
        const int rc = prefill_attn_kv_cache_update(h, in_dtype, batch, seq_len, k_new, v_new, pos_offsets, kv_map,
                                                    map_stride, k_cache, v_cache, n_slots, stream);
        if (rc != PA_OK) return rc;
        return prefill_attn_run_cached(h, in_dtype, batch, seq_len, q, k_cache, v_cache, n_slots, kv_map, map_stride,
                                       pos_offsets, out, score_scale, stream);
    }
    return splitk_impl(h, in_dtype, batch, seq_len, q, k_new, v_new, k_cache, v_cache, n_slots, kv_map, map_stride,
                       pos_offsets, out, score_scale, n_split, workspace, workspace_bytes, stream);
}

namespace {

constexpr int kDecodeCUs = 256;
constexpr int kDecodeMinKeysPerSplit = 256;

size_t decode_ws_bytes(const prefill_attn* h, int batch, int n_split) {
    return static_cast<size_t>(batch) * h->n_heads * n_split * (h->head_dim + 2) * sizeof(float);
}

}  // namespace

extern "C" size_t prefill_attn_decode_workspace_size(const prefill_attn* h, int batch, int n_split) {
    if (!h || batch < 0 || n_split < 1) return 0;
    return n_split == 1 ? 0 : decode_ws_bytes(h, batch, n_split);
}

namespace {

// Decode with the partials in `workspace` (workspace_bytes long).  strict: an
// explicit n_split whose partials do not fit is an error (PA_ETOOBIG) instead
// of being lowered.
int decode_impl(const prefill_attn* h, int in_dtype, int batch, const void* q, const void* k_cache,
                const void* v_cache, int n_slots, const int32_t* kv_map, int map_stride, const int32_t* pos_offsets,
                float* out, float score_scale, int n_split, void* workspace, size_t workspace_bytes, bool strict,
                void* stream) {
    if (!h || batch < 0 || n_split < 0) return PA_EINVAL;
    if (in_dtype != PA_IN_F32 && in_dtype != PA_IN_BF16) return PA_EINVAL;
    if (!std::isfinite(score_scale)) return PA_EINVAL;
    if (pos_offsets && !aligned4(pos_offsets)) return PA_EINVAL;
    if (batch == 0) return PA_OK;
    const int el = in_dtype == PA_IN_F32 ? 4 : 2;
    int rc = check_cache(h, el, 1, n_slots, kv_map, map_stride, k_cache, v_cache);
    if (rc != PA_OK) return rc;
    if (!q || !out || !aligned16(q) || !aligned16(out)) return PA_EINVAL;
    if (workspace && !aligned16(workspace)) return PA_EINVAL;

    const int G = pa::decode_group(h->n_heads, h->n_kv_heads);
    const int groups = batch * (h->n_heads / G);
    if (n_split == 0) {
        // One full round of resident workgroups: four per CU (two for eight heads per group).
        const int target = kDecodeCUs * (G >= 8 ? 2 : 4);
        n_split = std::max(1, target / groups);
        n_split = std::min(n_split, std::max(1, map_stride / kDecodeMinKeysPerSplit));
    } else if (strict && n_split > 1 && decode_ws_bytes(h, batch, n_split) > workspace_bytes) {
        return PA_ETOOBIG;
    }
    if (n_split > 1 && (!workspace || workspace_bytes < decode_ws_bytes(h, batch, 2))) n_split = 1;
    while (n_split > 1 && decode_ws_bytes(h, batch, n_split) > workspace_bytes) --n_split;

    pa::DecodeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.kv_map = kv_map;
    a.pos_offsets = pos_offsets;
    a.out = out;
    a.rope_f32 = h->d_rope_f32;
    a.status = h->d_status;
    a.ws = static_cast<float*>(workspace);
    a.batch = batch;
    a.n_heads = h->n_heads;
    a.n_kv_heads = h->n_kv_heads;
    a.max_seq = h->max_seq;
    a.map_stride = map_stride;
    a.n_slots = n_slots;
    a.n_split = n_split;
    const float scale = score_scale != 0.0f ? score_scale : 1.0f / std::sqrt(static_cast<float>(h->head_dim));
    a.logit_scale = scale * 1.44269504088896340736f;
    hipError_t e = pa::launch_decode(h->head_dim, in_dtype == PA_IN_F32, a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ELAUNCH;
}

}  // namespace

extern "C" int prefill_attn_decode(const prefill_attn* h, int in_dtype, int batch, const void* q,
                                   const void* k_cache, const void* v_cache, int n_slots, const int32_t* kv_map,
                                   int map_stride, const int32_t* pos_offsets, float* out, float score_scale,
                                   int n_split, void* workspace, size_t workspace_bytes, void* stream) {
    return decode_impl(h, in_dtype, batch, q, k_cache, v_cache, n_slots, kv_map, map_stride, pos_offsets, out,
                       score_scale, n_split, workspace, workspace_bytes, false, stream);
}

extern "C" int prefill_attn_decode_noalloc(const prefill_attn* h, int in_dtype, int batch, const void* q,
                                           const void* k_cache, const void* v_cache, int n_slots,
                                           const int32_t* kv_map, int map_stride, const int32_t* pos_offsets,
                                           float* out, float score_scale, int n_split, void* stream) {
    if (!h) return PA_EINVAL;
    float* scratch = nullptr;
    if (pa::noalloc_scratch(&scratch) != hipSuccess) return PA_ELAUNCH;
    return decode_impl(h, in_dtype, batch, q, k_cache, v_cache, n_slots, kv_map, map_stride, pos_offsets, out,
                       score_scale, n_split, scratch, pa::kNoAllocScratchBytes, true, stream);
}

extern "C" size_t prefill_attn_decode_noalloc_scratch_bytes(void) { return pa::kNoAllocScratchBytes; }

extern "C" int prefill_attn_device_peak(double* tflops, double* clock_ghz, void* stream) {
    if (!tflops || !clock_ghz) return PA_EINVAL;
    *tflops = 0.0;
    *clock_ghz = 0.0;
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return PA_EDEVICE;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return PA_EDEVICE;
    const hipError_t e = pa::measure_device_peak(60000, tflops, clock_ghz, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ELAUNCH;
}

extern "C" int prefill_attn_ring_map(int n_slots, int start, int count, int32_t* map) {
    if (n_slots < 1 || start < 0 || start >= n_slots || count < 0 || (count > 0 && !map)) return PA_EINVAL;
    for (int j = 0; j < count; ++j) map[j] = static_cast<int32_t>((static_cast<long long>(start) + j) % n_slots);
    return PA_OK;
}

extern "C" int prefill_attn_paged_map(const int32_t* block_table, int n_blocks, int block_size, int count,
                                      int32_t* map) {
    if (block_size < 1 || count < 0 || n_blocks < 0) return PA_EINVAL;
    if (count == 0) return PA_OK;
    if (!block_table || !map || (count - 1) / block_size >= n_blocks) return PA_EINVAL;
    for (int j = 0; j < count; ++j) {
        const long long blk = block_table[j / block_size];
        const long long slot = blk * block_size + j % block_size;
        if (blk < 0 || slot > 0x7fffffffLL) return PA_EINVAL;
        map[j] = static_cast<int32_t>(slot);
    }
    return PA_OK;
}

extern "C" int prefill_attn_status(prefill_attn* h, void* stream) {
    if (!h) return PA_EINVAL;
    if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return PA_ELAUNCH;
    int flag = 0;
    if (hipMemcpy(&flag, h->d_status, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return PA_ELAUNCH;
    if (flag != 0 && hipMemset(h->d_status, 0, sizeof(int)) != hipSuccess) return PA_ELAUNCH;
    if (hipDeviceSynchronize() != hipSuccess) return PA_ELAUNCH;
    return (flag & 1) ? PA_ERANGE : (flag & 2) ? PA_EOVERFLOW : PA_OK;
}

extern "C" int prefill_attn_destroy(prefill_attn* h) {
    if (!h) return PA_OK;
    const bool ok = hipDeviceSynchronize() == hipSuccess;
    free_handle(h);
    return ok ? PA_OK : PA_ELAUNCH;
}

extern "C" const char* prefill_attn_strerror(int code) {
    switch (code) {
        case PA_OK: return "success";
        case PA_EINVAL: return "invalid argument";
        case PA_ENOMEM: return "out of memory";
        case PA_EDEVICE: return "no usable gfx950 device";
        case PA_ELAUNCH: return "HIP runtime error";
        case PA_ERANGE: return "position outside the RoPE table or the index map, or a slot outside the cache";
        case PA_ETOOBIG: return "the requested split does not fit the fixed scratch of the no-allocation call";
        case PA_EOVERFLOW:
            return "an input value left the range the kernel computes in (fp16 operands of the bf16 path, "
                   "int8 digits of the int16 path); the output is not valid";
        default: return "unknown status code";
    }
}

extern "C" int prefill_attn_debug_rope_i16(const prefill_attn* h, int batch, int seq_len, const int16_t* x,
                                           int n_heads_x, const int32_t* pos_offsets, int16_t* x_rot,
                                           void* stream) {
    pa::RunArgs a;
    const int rc = prepare(h, batch, seq_len, pos_offsets, a);
    if (rc != PA_OK) return rc;
    if (n_heads_x < 1) return PA_EINVAL;
    if (batch == 0 || seq_len == 0) return PA_OK;
    if (!x || !x_rot || !aligned16(x) || !aligned16(x_rot)) return PA_EINVAL;
    a.q = x;
    hipError_t e = pa::launch_debug_rope_i16(h->head_dim, a, n_heads_x, x_rot, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ELAUNCH;
}

namespace {
int debug_scores(const prefill_attn* h, bool quant, int batch, int seq_len, const void* q, const void* k,
                 const int32_t* pos_offsets, int32_t* scores, void* stream) {
    pa::RunArgs a;
    const int rc = prepare(h, batch, seq_len, pos_offsets, a);
    if (rc != PA_OK) return rc;
    if (batch == 0 || seq_len == 0) return PA_OK;
    if (!q || !k || !scores || !aligned16(q) || !aligned16(k) || !aligned16(scores)) return PA_EINVAL;
    a.q = q;
    a.k = k;
    a.v = k;  // the score-export launch reads a V tensor of K's shape; its values do not reach the scores
    a.score_scale = 1.0f;
    hipError_t e = quant ? pa::launch_debug_scores_q16(h->head_dim, a, scores, static_cast<hipStream_t>(stream))
                         : pa::launch_debug_scores_i32(h->head_dim, a, scores, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ELAUNCH;
}
}  // namespace

extern "C" int prefill_attn_debug_scores_q16(const prefill_attn* h, int batch, int seq_len, const void* q,
                                             const void* k, const int32_t* pos_offsets, int32_t* scores,
                                             void* stream) {
    return debug_scores(h, true, batch, seq_len, q, k, pos_offsets, scores, stream);
}

extern "C" int prefill_attn_debug_scores_i32(const prefill_attn* h, int batch, int seq_len, const int16_t* q,
                                             const int16_t* k, const int32_t* pos_offsets, int32_t* scores,
                                             void* stream) {
    return debug_scores(h, false, batch, seq_len, q, k, pos_offsets, scores, stream);
}
