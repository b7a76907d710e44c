/*
 * prefill_attn.h -- fused RoPE causal prefill attention for AMD MI355X (gfx950).
 *
 * One call computes, for every batch element b, query head h and query token i,
 *
 *     O[b,i,h,:] = sum_{j<=i} softmax_j( RoPE(Q[b,i,h,:]) . RoPE(K[b,j,kvh(h),:]) * scale ) V[b,j,kvh(h),:]
 *
 * in a single kernel launch: RoPE is applied to Q and K inside the kernel from
 * cos/sin tables built once at init, the causal Q.K^T is computed tile by tile,
 * the softmax is evaluated blockwise with a running max and sum, and P.V is
 * accumulated, so no S x S score matrix is ever written to memory.
 *
 * Sources (page title and section):
 *  - "手写内核实现6倍prefill加速：边缘LLM推理的内存与计算协同优化"
 *    (www.0539edu.com/news/6082052): §2.2 one kernel fuses RoPE, Q.K^T, mask,
 *    softmax and the P.V product; §3.1 RoPE as a complex multiply with cos/sin
 *    tables indexed by position, done inside the Q.K^T loop; §2.2 all memory
 *    reserved once at start-up, none during a run.
 *  - the 2kiu.com/news/6082051 retelling of the same engine: §1.2 the three-call
 *    C interface (init / run / cleanup); §2.1 blocked attention with a constant
 *    working set and no S x S matrix; §3.3 int16 fixed-point RoPE tables.
 *  - the MNN-on-K3 blog (zhaode.wang/blog/2026/mnn-k3-riscv), §六: fused
 *    attention as blocked online softmax.
 *  - the XNet-DNN article (www.szyisi.cn/article/817147.html), §三.3
 *    FlashAttention-2: online softmax with the rescale deferred to the end.
 *
 * Conventions shared by every call:
 *  - Every function returns PA_OK (0) or a negative PA_E* code; nothing throws
 *    across this interface.
 *  - Tensors are dense row-major: Q [batch][seq_len][n_heads][head_dim],
 *    K and V [batch][seq_len][n_kv_heads][head_dim], O [batch][seq_len][n_heads][head_dim].
 *  - Query head h reads KV head kvh(h) = h / (n_heads / n_kv_heads) (contiguous
 *    groups, the repeat-interleave convention for grouped-query attention).
 *  - RoPE rotates adjacent pairs (x, y) = (X[2k], X[2k+1]) by the angle
 *    p * theta_k, theta_k = rope_theta^(-2k/head_dim), where p = pos_offsets[b] + i
 *    is the position of token i of batch element b (queries and keys alike; the
 *    causal mask stays j <= i).
 *  - Device pointers must belong to the device that was current at init and be
 *    16-byte aligned.  The caller owns Q, K, V, O, pos_offsets and the stream;
 *    the handle owns its device tables and its status word.
 */
#ifndef PREFILL_ATTN_H
#define PREFILL_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct prefill_attn prefill_attn; /* opaque handle */

/* Input element types accepted by prefill_attn_run. */
enum prefill_attn_dtype {
    PA_IN_F32 = 0,  /* Q, K, V float32; products on the fp32 matrix cores */
    PA_IN_BF16 = 1, /* Q, K, V bfloat16; rotated Q'/K', P and V rounded to fp16 for the matrix cores, fp32
                       accumulate.  Range: V, K' = RoPE(K) and Q' = RoPE(Q) * score_scale * log2(e) must
                       stay below 65504 in magnitude (every |x| < 2^15 is enough while score_scale <= 0.5);
                       values below 2^-14 keep fewer bits (fp16 subnormals).  A larger K' or a non-finite O
                       sets the status word (PA_EOVERFLOW from prefill_attn_status). */
    PA_IN_I16 = 2,  /* Q, K int16 fixed point, V bfloat16; integer RoPE, exact int32 scores, fp32 softmax.
                       Range: every rotated Q'/K' value must lie in [-16448, 16319] (the int8 digit split
                       of the scores; |x| <= 11500 for every input is enough); outside it the scores are
                       wrong and the status word is set (PA_EOVERFLOW).  Every score Q'.K' must also fit
                       int32, or it wraps unreported (|x| <= 2895 for every input is enough at head_dim
                       128).  V as for PA_IN_BF16. */
    PA_IN_BF16_Q16 = 3, /* Q, K, V bfloat16; each (token, head) row of Q and K quantised inside the kernel to
                          int16 codes, round-half-even(x * 2047 / max|x|) in fp32 (the 2kiu.com retelling, §3.3:
                          per-token dynamic activation scale), then the PA_IN_I16 path with
                          logit = (int32 score) * score_scale * (max|q| / 2047) * (max|k| / 2047) */
    PA_IN_I16_PWL = 4  /* as PA_IN_I16, with the softmax of the 2kiu.com retelling, §3.3: exp of
                          x = logit - (row max) as the chord of e^x between the integer knots floor(x) and
                          floor(x) + 1 (16 unit segments on [-8, 8)), 0 below -8, and the normalisation by
                          a Newton-Raphson reciprocal (seed 48/17 - 32/17 f, three steps); the row max comes
                          from a first pass over the keys.  prefill_attn_run only. */
};

enum prefill_attn_status {
    PA_OK = 0,
    PA_EINVAL = -1,  /* bad argument: shape, NULL or misaligned pointer, unknown dtype */
    PA_ENOMEM = -2,  /* device or host allocation failed (init only) */
    PA_EDEVICE = -3, /* no device, or the current device is not gfx950 */
    PA_ELAUNCH = -4, /* the HIP runtime rejected a launch or a copy */
    PA_ERANGE = -5,  /* a run saw pos_offsets[b] < 0 or pos_offsets[b] + seq_len > max_seq (or, for the
                        cache calls, beyond map_stride, or a map entry outside the cache) */
    PA_ETOOBIG = -6, /* prefill_attn_decode_noalloc: the requested split's partials exceed the
                        library's fixed scratch */
    PA_EOVERFLOW = -7 /* a run saw a value outside the range its kernel computes in: a non-finite
                         O (bf16 path: an fp16 operand overflowed, or an input was not finite) or an
                         fp16 K' = RoPE(K) beyond 65504, or (int16 path) a rotated Q'/K' value outside
                         [-16448, 16319], where the int8 digit split wraps; O is not valid */
};

/*
 * Create a handle for one attention shape on the current HIP device.
 *   n_heads     query heads, >= 1
 *   n_kv_heads  key/value heads, >= 1, dividing n_heads
 *   head_dim    64, 96 or 128
 *   max_seq     largest position + 1 any run may use (table rows), 1 .. 1048576
 *   rope_theta  RoPE base, > 1
 * Builds the RoPE cos/sin tables on the host in fp64 (each value rounded once, to
 * fp32 pairs for the fp32 and bf16 paths and decode, and to Q1.14 int16 pairs
 * for the int16 paths), copies them to the device and
 * allocates the status word.  All allocation happens here; prefill_attn_run
 * allocates nothing.
 * On success *out receives the handle; on failure *out is set to NULL.
 */
int prefill_attn_init(prefill_attn** out, int n_heads, int n_kv_heads, int head_dim,
                      int max_seq, double rope_theta);

/*
 * Enqueue one fused attention pass on `stream` (a hipStream_t; NULL = the null
 * stream).  Asynchronous: returns once the kernel is queued; no host sync, no
 * allocation, no memset, so the call may be captured into a HIP graph.
 *   in_dtype     a prefill_attn_dtype value
 *   batch        >= 0; seq_len in 0 .. max_seq (batch == 0 or seq_len == 0 is a no-op)
 *   q, k, v      device tensors in the layouts above, of in_dtype (V is bf16 for PA_IN_I16)
 *   pos_offsets  device int32[batch], or NULL for all zeros
 *   out          device float32 O; every element of rows i < seq_len is written
 *   score_scale  multiplies the score: PA_IN_F32/PA_IN_BF16 logit = (Q'.K') * score_scale,
 *                PA_IN_I16 logit = (int32 score) * score_scale, PA_IN_BF16_Q16 as documented
 *                with the enum; 0 selects 1/sqrt(head_dim)
 * A batch element whose positions leave [0, max_seq) gets O = 0 and sets the
 * handle's status word (read it with prefill_attn_status).  Runs on one handle
 * may overlap on several streams; they share only that status word.
 */
int prefill_attn_run(const prefill_attn* h, int in_dtype, int batch, int seq_len,
                     const void* q, const void* k, const void* v,
                     const int32_t* pos_offsets, float* out, float score_scale,
                     void* stream);

/*
 * KV-prefix (chunked) prefill against a KV cache.
 *
 * Sources: the page titled "手写内核实现6倍prefill加速", §2.2 (the cache-update
 * kernel copies only the K/V of the new tokens and leaves older entries in
 * place) and §3.2 (ring KV cache: K/V stored wherever there is room, with an
 * index map holding one physical offset per logical position, so attention
 * still reads the keys in logical order); the 2kiu.com retelling, §3.4 (a
 * ring of fixed slots indexed with a wrap-around).
 *
 * A cache is a pair of device tensors K_cache, V_cache [n_slots][n_kv_heads][head_dim]
 * owned by the caller (element type as for prefill_attn_run: f32, bf16, or
 * int16 K with bf16 V).  kv_map is a device int32 [batch][map_stride]:
 * kv_map[b*map_stride + j] is the slot holding logical position j of
 * sequence b.  pos_offsets[b] (NULL = all 0) is the number of positions the
 * cache already holds for sequence b, so the chunk's token i has logical
 * position and RoPE position pos_offsets[b] + i.
 *
 * prefill_attn_kv_cache_update: copies K_new, V_new [batch][seq_len][n_kv_heads][head_dim]
 *   (token i of sequence b) into slot kv_map[b*map_stride + pos_offsets[b] + i] of
 *   the caches.  Nothing else is written.  The slots the new tokens map to must be
 *   distinct (otherwise which write lands is unspecified).
 * prefill_attn_run_cached: for the chunk's queries Q [batch][seq_len][n_heads][head_dim],
 *     O[b,i,h,:] = sum_{j <= P+i} softmax_j( RoPE_{P+i}(Q[b,i,h]) . RoPE_j(Kc[map(b,j), kvh(h)]) * scale ) Vc[map(b,j), kvh(h)]
 *   with P = pos_offsets[b] and map(b,j) = kv_map[b*map_stride + j]: keys are read
 *   through the index map in logical order and rotated at their logical position,
 *   inside the same fused kernel as prefill_attn_run.  The chunk's own K/V must
 *   already be in the cache (call prefill_attn_kv_cache_update first, on the same
 *   stream).  With pos_offsets all 0 and the identity map this is prefill_attn_run.
 * Both: asynchronous on `stream`, no allocation.  PA_EINVAL for a bad shape or
 *   pointer: n_slots < 1, map_stride < max(1, seq_len), a cache larger than
 *   2^32 - 1 bytes, NULL or misaligned pointers (caches, Q, K_new, V_new, out 16-byte,
 *   kv_map and pos_offsets 4-byte aligned), an unknown dtype.  On the device, a
 *   sequence with pos_offsets[b] < 0 or pos_offsets[b] + seq_len > map_stride
 *   (for the run also > max_seq) is skipped (run: O = 0) and a map entry outside
 *   [0, n_slots) is read as slot 0 (update: skipped); both set the status word
 *   (PA_ERANGE from prefill_attn_status).  The caller owns caches, map and offsets.
 */
int prefill_attn_kv_cache_update(const prefill_attn* h, int in_dtype, int batch, int seq_len,
                                 const void* k_new, const void* v_new, const int32_t* pos_offsets,
                                 const int32_t* kv_map, int map_stride,
                                 void* k_cache, void* v_cache, int n_slots, void* stream);
int prefill_attn_run_cached(const prefill_attn* h, int in_dtype, int batch, int seq_len,
                            const void* q, const void* k_cache, const void* v_cache, int n_slots,
                            const int32_t* kv_map, int map_stride, const int32_t* pos_offsets,
                            float* out, float score_scale, void* stream);

/*
 * prefill_attn_run_cached_splitk: prefill_attn_run_cached with the keys of every
 * (query block, sequence, head) split over n_split workgroups, for chunks whose
 * prefix is long compared with the chunk (few query blocks, many keys each).
 * Each split writes an unnormalised partial (O, running max, sum) to `workspace`
 * (device, 16-byte aligned, caller-owned, at least
 * prefill_attn_run_cached_workspace_size(h, batch, seq_len, n_split) bytes) and a
 * second kernel merges them by the log-sum-exp rule (the same rule the XNet-DNN
 * article, §三.3, uses to combine blocks of the online softmax).  n_split = 0
 * lets the library choose; a NULL or short workspace lowers n_split to what fits,
 * down to 1, which is prefill_attn_run_cached.  PA_IN_F32 always runs unsplit.
 * n_split is an upper bound: each (query block, sequence, head) uses only as
 * many splits as give every split at least four 64-key tiles of its own keys.
 * The workspace contents are scratch between calls (nothing needs clearing).
 * Results equal prefill_attn_run_cached's up to the rounding of the merge.
 */
size_t prefill_attn_run_cached_workspace_size(const prefill_attn* h, int batch, int seq_len, int n_split);
int prefill_attn_run_cached_splitk(const prefill_attn* h, int in_dtype, int batch, int seq_len,
                                   const void* q, const void* k_cache, const void* v_cache, int n_slots,
                                   const int32_t* kv_map, int map_stride, const int32_t* pos_offsets,
                                   float* out, float score_scale, int n_split,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * prefill_attn_run_cached_update: prefill_attn_kv_cache_update followed by
 * prefill_attn_run_cached_splitk (n_split, workspace and their rules as
 * there; n_split = 1 is the unsplit prefill_attn_run_cached), as one launch
 * for the 16-bit input types: the attention reads the chunk's own keys
 * (logical positions pos_offsets[b] .. pos_offsets[b] + seq_len - 1) from
 * k_new / v_new ([batch][seq_len][n_kv_heads][head_dim], as for the update),
 * and the same launch writes those rows to their cache slots.  The update's
 * copy then costs no launch of its own and its rows are read once (the page
 * titled "手写内核实现6倍prefill加速", §2.2 and §3.2: the update copies only
 * the new tokens into the KV cache the attention reads through the index map).
 * Precondition beyond the update's: no slot that the chunk writes is the slot
 * of another logical position the chunk's queries attend to (the map is
 * one-to-one over positions 0 .. pos_offsets[b] + seq_len - 1).  Results equal
 * those of the two calls bit for bit; a chunk whose positions leave the table
 * or the map writes nothing and gets O = 0 (PA_ERANGE).  PA_IN_F32 runs the two
 * calls as two launches.
 */
int prefill_attn_run_cached_update(const prefill_attn* h, int in_dtype, int batch, int seq_len,
                                   const void* q, const void* k_new, const void* v_new,
                                   void* k_cache, void* v_cache, int n_slots,
                                   const int32_t* kv_map, int map_stride, const int32_t* pos_offsets,
                                   float* out, float score_scale, int n_split,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode attention: one new token per sequence against the KV cache.
 *
 * Sources: the page titled "手写内核实现6倍prefill加速", §3.1 (RoPE from
 * position-indexed tables) and §3.2 (keys read through the index map in
 * logical order); the MNN-on-K3 blog (zhaode.wang/blog/2026/mnn-k3-riscv),
 * §五 and §六: decode attention is a short matrix-vector product limited by
 * memory bandwidth, computed as blocked online softmax.
 *
 * For sequence b, with P = pos_offsets[b] (NULL = all 0) the position of its
 * new token, whose K/V must already be in the cache at logical position P:
 *     out[b,h,:] = sum_{j <= P} softmax_j( RoPE_P(q[b,h]) . RoPE_j(Kc[map(b,j), kvh(h)]) * scale ) Vc[map(b,j), kvh(h)]
 * i.e. prefill_attn_run_cached with seq_len = 1.  q is [batch][n_heads][head_dim],
 * out [batch][n_heads][head_dim] float32, caches and kv_map as for the cache calls
 * above.  in_dtype is PA_IN_F32 or PA_IN_BF16 (caches of the same type); all
 * arithmetic is fp32.
 *
 * The keys of a sequence are split over n_split workgroups (0 = chosen by the
 * library so that about a thousand workgroups run); with n_split > 1 the partial
 * results go to `workspace` (device, 16-byte aligned, caller-owned, at least
 * prefill_attn_decode_workspace_size(h, batch, n_split) bytes) and a second
 * kernel merges them.  If the workspace is NULL or too small the call uses the
 * largest split it can hold (n_split = 1 needs none).  Asynchronous, no
 * allocation.  PA_EINVAL for bad shapes or pointers as for the cache calls; a
 * sequence with P < 0, P + 1 > map_stride or P + 1 > max_seq gets out = 0 and
 * sets the status word, as does a map entry outside [0, n_slots) (read as slot 0).
 */
size_t prefill_attn_decode_workspace_size(const prefill_attn* h, int batch, int n_split);
int prefill_attn_decode(const prefill_attn* h, int in_dtype, int batch, const void* q,
                        const void* k_cache, const void* v_cache, int n_slots,
                        const int32_t* kv_map, int map_stride, const int32_t* pos_offsets,
                        float* out, float score_scale, int n_split,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * prefill_attn_decode_noalloc: prefill_attn_decode for callers that cannot
 * allocate device memory or pass a workspace -- code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The split partials go
 * to a scratch array that the library holds in device memory, one copy per
 * device, from the first call on that device (init looks it up for the
 * current device) until the process ends.  The call allocates nothing, also
 * not through a library.
 *
 * Arguments, results, status and errors are prefill_attn_decode's, less the
 * workspace.  The scratch holds prefill_attn_decode_noalloc_scratch_bytes()
 * bytes (8 MiB): n_split = 0 chooses the split as prefill_attn_decode does and
 * lowers it to what fits (down to 1, which uses no scratch); an explicit
 * n_split > 1 whose partials, prefill_attn_decode_workspace_size(h, batch,
 * n_split) bytes, exceed the scratch returns PA_ETOOBIG and enqueues nothing.
 * The scratch needs no clearing (each split writes its partial before the merge
 * reads it), but all calls on one device share it: two calls that may run at
 * the same time on that device (other streams, other threads) race and give
 * wrong results.  Calls on one stream are ordered and safe.
 */
int prefill_attn_decode_noalloc(const prefill_attn* h, int in_dtype, int batch, const void* q,
                                const void* k_cache, const void* v_cache, int n_slots,
                                const int32_t* kv_map, int map_stride, const int32_t* pos_offsets,
                                float* out, float score_scale, int n_split, void* stream);
size_t prefill_attn_decode_noalloc_scratch_bytes(void);

/*
 * Device characterisation (not part of the attention path): the measured
 * matrix-core peak of the current device in TFLOP/s (v_mfma_f32_32x32x16_f16
 * on every CU, four independent accumulators per wave, two waves per SIMD,
 * operands varying lane by lane, over a launch of about 10 ms) and the shader
 * clock it held in GHz (shader-clock over real-time counter),
 * the roofline denominators reported beside the vendor peak (the XNet-DNN
 * article, §三: kernels measured against a micro-benchmarked roofline).
 * Synchronous; allocates and frees a few KB of device memory; under a second.
 * PA_EDEVICE if the current device is not gfx950.
 */
int prefill_attn_device_peak(double* tflops, double* clock_ghz, void* stream);

/*
 * Host-only index-map builders (caller-owned host arrays; copy the result to the
 * device row of the sequence).
 *   prefill_attn_ring_map:  map[j] = (start + j) mod n_slots, j < count (a ring of
 *     n_slots slots whose oldest live position sits at `start`); needs n_slots >= 1,
 *     0 <= start < n_slots, count >= 0.
 *   prefill_attn_paged_map: map[j] = block_table[j / block_size] * block_size + j % block_size,
 *     j < count (the cache cut into blocks of block_size slots, block_table[n] the
 *     physical block of logical block n); needs block_size >= 1, n_blocks blocks
 *     covering count positions, non-negative blocks and slots below 2^31.
 */
int prefill_attn_ring_map(int n_slots, int start, int count, int32_t* map);
int prefill_attn_paged_map(const int32_t* block_table, int n_blocks, int block_size, int count, int32_t* map);

/*
 * Synchronise `stream`, then report and clear the status word: PA_ERANGE if any
 * call since the last status call saw an out-of-range position, map row or
 * slot, else PA_EOVERFLOW if one saw a value outside its kernel's range (see
 * PA_EOVERFLOW and the input types), else PA_OK.
 */
int prefill_attn_status(prefill_attn* h, void* stream);

/* Free everything init allocated.  NULL-safe.  Synchronises the device first. */
int prefill_attn_destroy(prefill_attn* h);

/* Static English text for a status code. */
const char* prefill_attn_strerror(int code);

/*
 * Host-only RoPE table builders (no device needed), the same code init uses.
 * Row p, pair k of the result holds the angle a = p * rope_theta^(-2k/head_dim),
 * evaluated in fp64:
 *   _f32: out[(p*head_dim/2 + k)*2 + 0] = (float)cos(a), [... + 1] = (float)sin(a)
 *         (round to nearest even), out has max_seq*head_dim floats;
 *   _q14: out[(p*head_dim/2 + k)*2 + 0] = round(cos(a) * 2^14), [... + 1] = round(sin(a) * 2^14)
 *         (nearest, ties away from zero), out has max_seq*head_dim int16.
 * head_dim must be even and positive, max_seq positive; out is caller-owned host memory.
 */
int prefill_attn_rope_table_f32(int max_seq, int head_dim, double rope_theta, float* out);
int prefill_attn_rope_table_q14(int max_seq, int head_dim, double rope_theta, int16_t* out);

/*
 * Test exports for the int16 variant, run by the device code of PA_IN_I16:
 *   prefill_attn_debug_rope_i16: x [batch][seq_len][n_heads_x][head_dim] int16 ->
 *     x_rot (same shape) = (x C - y S + 2^13) >> 14, (x S + y C + 2^13) >> 14 at
 *     position pos_offsets[b] + i (the fixed-point rotation of the page titled
 *     "手写内核实现6倍prefill加速", §3.1, with Q1.14 tables), formed by the K staging
 *     of the int16 kernels (table addressing, rotation, digit split into LDS) with
 *     the staging width a prefill of this shape uses, and read back as 128 h + l
 *     from the digit planes.  Values outside [-16448, 16319] set the status word
 *     (PA_EOVERFLOW) and come back wrong.
 *   prefill_attn_debug_scores_i32: the int32 scores of the causal part,
 *     scores[b][h][i][j] = Q'[b,i,h] . K'[b,j,kvh(h)] for j <= i, of
 *     scores[batch][n_heads][seq_len][seq_len] (entries j > i are not written),
 *     stored by the very kernel prefill_attn_run launches for PA_IN_I16 at this
 *     shape (eight-wave two-group or four-wave, the int8 digit-split matrix-core
 *     path) from a debug instantiation that adds the store and writes no O.
 * Same pointer, alignment and stream rules as prefill_attn_run.
 */
int prefill_attn_debug_rope_i16(const prefill_attn* h, int batch, int seq_len,
                                const int16_t* x, int n_heads_x, const int32_t* pos_offsets,
                                int16_t* x_rot, void* stream);
int prefill_attn_debug_scores_i32(const prefill_attn* h, int batch, int seq_len,
                                  const int16_t* q, const int16_t* k, const int32_t* pos_offsets,
                                  int32_t* scores, void* stream);
/* The same causal scores for bfloat16 Q/K through the kernel of PA_IN_BF16_Q16
 * (in-kernel quantisation): scores of the int16 codes. */
int prefill_attn_debug_scores_q16(const prefill_attn* h, int batch, int seq_len,
                                  const void* q, const void* k, const int32_t* pos_offsets,
                                  int32_t* scores, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PREFILL_ATTN_H */
