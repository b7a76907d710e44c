// Internal interface between the C-ABI layer (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Everything one fused attention launch needs.  Pointers are device pointers.
struct RunArgs {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* pos_offsets;  // may be null: all offsets 0
    float* out;
    const float* rope_f32;       // [max_seq][head_dim/2] (cos, sin) fp32 pairs
    const int16_t* rope_q14;     // [max_seq][head_dim/2] (C, S) Q1.14 pairs
    int* status;                 // bit 0: a position left the table or map; bit 1: a value left its range
    int batch;
    int seq_len;
    int n_heads;
    int n_kv_heads;
    int max_seq;
    float score_scale;           // resolved (never 0 here)
    // Cached prefill only (kv_map non-null): k and v are caches [n_slots][n_kv_heads][D],
    // kv_map[b * map_stride + j] is the slot of logical position j of sequence b, and
    // pos_offsets[b] is the number of positions the cache held before this chunk.
    const int32_t* kv_map;
    int map_stride;
    int n_slots;
    // Split-K (cached prefill only): the keys of every (query block, sequence,
    // head) are divided over n_split workgroups, each writing its unnormalised
    // O and (max, sum) to ws: [rows][n_split][D] fp32, then [rows][n_split][2],
    // rows = batch * seq_len * n_heads in the order of O.
    int n_split;
    float* ws;
    // Paired launch (unsplit eight-wave kernels): workgroup (j, batch, head)
    // runs query block n_qblocks - 1 - j and then block j, so every pair
    // covers the same number of key tiles.
    int paired;
    // Score-export launches of the int16 paths only: [batch][n_heads][S][S] int32
    // scores of every key at or before its query (no O is written).
    int32_t* dbg_scores;
    // Cached prefill with the chunk's own K/V (mapped, 16-bit types): the
    // chunk's keys are read from these [batch][seq_len][n_kv_heads][D]
    // tensors, and the launch writes them to their cache slots in k / v.
    const void* k_new;
    const void* v_new;
};

hipError_t launch_attn_bf16(int head_dim, const RunArgs& a, hipStream_t stream);
hipError_t launch_attn_f32(int head_dim, const RunArgs& a, hipStream_t stream);
hipError_t launch_attn_i16(int head_dim, const RunArgs& a, hipStream_t stream);
// bf16 Q/K quantised in-kernel per (token, head) row to int16, then the int16 path.
hipError_t launch_attn_i16q(int head_dim, const RunArgs& a, hipStream_t stream);
// int16 Q/K with the piecewise-linear softmax and Newton reciprocal (two passes).
hipError_t launch_attn_i16pwl(int head_dim, const RunArgs& a, hipStream_t stream);

// Copies the new tokens' K/V ([batch][seq_len][n_kv_heads][D], `el` bytes per
// element) into their cache slots; a.k/a.v are the new K/V, dst_k/dst_v the caches.
hipError_t launch_kv_cache_update(int head_dim, int el, const RunArgs& a, void* dst_k, void* dst_v,
                                  hipStream_t stream);

// Decode attention (one new token per sequence) against a KV cache.
struct DecodeArgs {
    const void* q;               // [batch][n_heads][D]
    const void* k;               // caches [n_slots][n_kv_heads][D]
    const void* v;
    const int32_t* kv_map;       // [batch][map_stride] logical position -> slot
    const int32_t* pos_offsets;  // [batch] position of the new token (may be null: 0)
    float* out;                  // [batch][n_heads][D]
    const float* rope_f32;
    int* status;
    float* ws;                   // n_split > 1: partial O, then (max, sum) pairs
    int batch;
    int n_heads;
    int n_kv_heads;
    int max_seq;
    int map_stride;
    int n_slots;
    int n_split;
    float logit_scale;           // score_scale * log2(e)
};

// Merge of split-K partials: out[r][:] = sum_s w_s O_s / sum_s w_s l_s over the
// rows r < a.batch * a.n_heads (DecodeArgs.batch counts row groups of n_heads).
hipError_t launch_split_merge(int head_dim, const DecodeArgs& a, hipStream_t stream);
// Compute units of the current device (cached per device).
int device_cus();
// Whether an eight-wave launch of `rows`-row query blocks (head_pack query
// heads per workgroup) runs as pairs of blocks (n-1-j, j).
bool use_pairs(const RunArgs& a, int rows = 256, int head_pack = 1);
// Whether a cached-prefill launch of this shape uses eight-wave workgroups.
bool prefill_uses_eight_waves(const RunArgs& a);

// Query heads served by one decode workgroup (a divisor of n_heads / n_kv_heads).
int decode_group(int n_heads, int n_kv_heads);
hipError_t launch_decode(int head_dim, bool f32, const DecodeArgs& a, hipStream_t stream);

// Fixed scratch of the no-allocation decode call (split partials), in bytes.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
// Device address of that scratch on the current device; the symbol lookup
// runs once per device (init, or the first call on another device).
hipError_t noalloc_scratch(float** ptr);

// Matrix-core peak (TFLOP/s of v_mfma_f32_32x32x16_f16, every CU busy) and the
// shader clock of the current device, measured by one timed launch of `iters`
// loop steps (allocates and synchronises: a characterisation call).
hipError_t measure_device_peak(int iters, double* tflops, double* clock_ghz, hipStream_t stream);

// Int16 test exports; RunArgs.q is the tensor to rotate (x) for the rope one,
// q/k for the scores one; `dst` receives int16 x_rot or int32 scores.
hipError_t launch_debug_rope_i16(int head_dim, const RunArgs& a, int n_heads_x, int16_t* dst,
                                 hipStream_t stream);
hipError_t launch_debug_scores_i32(int head_dim, const RunArgs& a, int32_t* dst, hipStream_t stream);
hipError_t launch_debug_scores_q16(int head_dim, const RunArgs& a, int32_t* dst, hipStream_t stream);

// Host: the fp32 and Q1.14 RoPE tables of init from one fp64 pass
// (each value rounded once, as the exported single-table builders do).
int build_rope_tables(int max_seq, int head_dim, double rope_theta, float* f32, int16_t* q14);

}  // namespace pa
