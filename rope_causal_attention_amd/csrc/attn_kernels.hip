// Fused RoPE causal prefill attention kernels for gfx950 (MI355X).
//
// What is computed (pages cited by title and section):
//  * "手写内核实现6倍prefill加速：边缘LLM推理的内存与计算协同优化", §2.2/§3.1:
//    one kernel applies RoPE to Q and K from position-indexed cos/sin tables
//    (a complex multiply on adjacent pairs), forms Q.K^T, applies the mask,
//    the softmax and the product with V; rotated K goes straight into the dot
//    product and is never written back to memory.
//  * 2kiu.com/news/6082051 retelling, §2.1: attention in blocks of Q rows and
//    K columns with a working set independent of the sequence length; §3.3:
//    int16 fixed-point RoPE tables and activations.
//  * MNN-on-K3 blog (zhaode.wang/blog/2026/mnn-k3-riscv), §六: QK, online
//    softmax and PV merged into one blocked pass; §三: an 8-bit operand split
//    into two narrower digits whose products recombine exactly.
//  * XNet-DNN article (www.szyisi.cn/article/817147.html), §三.3
//    FlashAttention-2: Q in the outer loop so work spreads over sequence
//    blocks, Q rows split across waves that share the K/V tiles, the rescale
//    by the running sum deferred to the end.
//
// gfx950 design (not a translation of the pages' CPU/NPU code):
//  * one workgroup = 4 waves x 32 query rows (BM = 128) of one (batch, head);
//    K/V tiles of 64 keys are staged in LDS, double-buffered, so the global
//    loads of tile t+1 are in flight while tile t is on the matrix cores;
//  * S^T = K'.Q'^T on v_mfma_f32_32x32x16_f16: each lane then owns one query
//    column and 16 keys of every 32x32 block, so the softmax row max / row sum
//    are in-lane plus one v_permlane32_swap between the two lane halves;
//  * the f16 probabilities stay in registers and feed O^T += V^T.P^T directly
//    as the B operand; V^T is written to LDS transposed (and with the key order
//    the accumulator layout implies) while V is converted bf16 -> f16;
//  * Q' is rotated once per workgroup, pre-multiplied by score_scale*log2(e)
//    and kept in registers for the whole key loop; exp2 replaces exp;
//  * the running max is only moved (and O, l rescaled) when it grows by more
//    than 2^8, which keeps the result exact (the same stale max is used for O
//    and for l) and skips almost every rescale;
//  * workgroups are ordered longest (most keys) first, and the (batch, head)
//    pairs are split over the 8 XCDs so one head's K/V stays in one L2.
//  * int16 variant: Q'/K' rotated in integers, split into signed 8-bit digits
//    a = 128 h + l (l in [-64, 63], h in [-23, 23] for |a| <= 2897), and the
//    exact int32 score is recombined from the v_mfma_i32_32x32x32_i8
//    products hh, ll and hl + lh (the two cross products share one
//    accumulator); P.V as in the bf16 kernel.
//  * fp32 variant: v_mfma_f32_32x32x2_f32 for both products, fp32 LDS tiles.

#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include "internal.h"
#include "device_common.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int BM = 32 * kWaves;  // query rows per workgroup
constexpr int kMinSplitTiles = 4;  // split-K: fewest key tiles per non-empty split
constexpr float kRescaleSlack = 8.0f;  // log2 units: P stays <= 2^8 between rescales

// Query i of the workgroup's (batch, head) has table position off + i.  Keys
// are numbered in key space: key j has table position koff + j, the keys a
// query i sees are j <= kshift + i, and there are NK = kshift + S keys.
//  * plain prefill: the keys are the same S tokens, koff = off, kshift = 0;
//  * cached prefill (MAPPED): the keys are logical positions 0 .. off + S - 1
//    of the cache, koff = 0, kshift = off (the tokens cached before the chunk).
struct Ctx {
    int b, hq, hkv, off, S, q0;
    int koff, kshift, NK;
    int split;  // this workgroup's key range among n_split (split-K only)
};

// Context of query block bp; false when the sequence's positions leave the table.
template <int BM, bool MAPPED>
__device__ __forceinline__ bool make_ctx_at(const RunArgs& a, const BlockPos& bp, int split, Ctx& c) {
    c.split = split;
    c.b = bp.b;
    c.hq = bp.hq;
    c.hkv = bp.hq / (a.n_heads / a.n_kv_heads);
    c.S = a.seq_len;
    c.q0 = bp.qb * BM;
    c.off = a.pos_offsets ? a.pos_offsets[bp.b] : 0;
    c.koff = MAPPED ? 0 : c.off;
    c.kshift = MAPPED ? c.off : 0;
    c.NK = c.kshift + c.S;
    const long long end = static_cast<long long>(c.off) + a.seq_len;
    return c.off >= 0 && end <= a.max_seq && (!MAPPED || end <= a.map_stride);
}

template <int BM, bool MAPPED, bool SPLIT = false>
__device__ __forceinline__ bool make_ctx(const RunArgs& a, Ctx& c) {
    const int n_qblocks = (a.seq_len + BM - 1) / BM;
    const int bid = SPLIT ? static_cast<int>(blockIdx.x) / a.n_split : static_cast<int>(blockIdx.x);
    const int split = SPLIT ? static_cast<int>(blockIdx.x) % a.n_split : 0;
    return make_ctx_at<BM, MAPPED>(a, map_block(n_qblocks, a.batch, a.n_heads, bid), split, c);
}

__device__ __forceinline__ size_t q_index(const RunArgs& a, const Ctx& c, int i, int D) {
    return ((static_cast<size_t>(c.b) * c.S + i) * a.n_heads + c.hq) * D;
}
__device__ __forceinline__ size_t kv_index(const RunArgs& a, const Ctx& c, int j, int D) {
    return ((static_cast<size_t>(c.b) * c.S + j) * a.n_kv_heads + c.hkv) * D;
}

// Rows of one (batch, head): a uniform base plus 32-bit byte offsets.
//  * plain: token j of a [B][S][H][D] tensor is at base + j * stride;
//  * mapped (cached prefill): logical key j is in cache slot map[j], at
//    base + map[j] * stride.  A slot outside [0, n_slots) reads slot 0 and
//    sets the status word, so a bad map never reads outside the cache.
struct Rows {
    const char* base;
    uint32_t stride;     // bytes between consecutive tokens / slots
    const int32_t* map;  // mapped only: this sequence's row of the index map
    int n_slots;
    int* status;
    // mapped, with the chunk's own K/V passed in (not yet in the cache):
    // logical key n_first + i is token i of the chunk, at nbase + i * stride
    const char* nbase;
    int n_first;

    // Base of the 64-key tile `tile`, and the offset of its row `row`.
    template <bool MAPPED>
    __device__ __forceinline__ const char* tile_base(int tile) const {
        return MAPPED ? base : base + static_cast<size_t>(tile * BN) * stride;
    }
    template <bool MAPPED>
    __device__ __forceinline__ uint32_t row_off(int tile, int row) const {
        if (!MAPPED) return static_cast<uint32_t>(row) * stride;
        int slot = map[tile * BN + row];
        if (static_cast<unsigned>(slot) >= static_cast<unsigned>(n_slots)) {
            atomicOr(status, 1);
            slot = 0;
        }
        return static_cast<uint32_t>(slot) * stride;
    }
    // Start of row `row` of tile `tile`.  Mapped: `pre`, when given, holds the
    // row's checked slot offset (as row_off forms it) read ahead of time, so
    // the row's load does not wait for its map entry.
    template <bool MAPPED>
    __device__ __forceinline__ const char* row_addr(int tile, int row, const uint32_t* pre = nullptr) const {
        if constexpr (!MAPPED) {
            return tile_base<false>(tile) + static_cast<uint32_t>(row) * stride;
        } else {
            const int j = tile * BN + row;
            if (nbase && j >= n_first) return nbase + static_cast<size_t>(j - n_first) * stride;
            return base + (pre ? *pre : row_off<true>(tile, row));
        }
    }
};
// Mapped launches: the map entries (unchecked slots) of the N key rows a
// thread stages from tile `tile` (row_of(n) is its n-th row; rows past the
// last key clamped to it as the clamped loads do; for a full tile the clamp
// changes nothing).  Nothing here uses the values, so their loads stay in
// flight beside the tile loads issued before them.  The entries of keys read
// from the chunk's own tensor are read too but not used (the cache update
// checks those).
template <int N, class RowOf>
__device__ __forceinline__ void read_slots(const Rows& p, int n_keys, int tile, uint32_t (&slot)[N], RowOf row_of) {
#pragma unroll
    for (int n = 0; n < N; ++n) slot[n] = p.map[min(tile * BN + row_of(n), n_keys - 1)];
}
// The slots' byte offsets; a slot outside [0, n_slots) reads slot 0 (as
// row_off) and sets `bad`, which the caller reports in the status word.
template <int N>
__device__ __forceinline__ void slot_offsets(const Rows& p, uint32_t (&slot)[N], bool& bad) {
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const bool ok = slot[n] < static_cast<uint32_t>(p.n_slots);
        bad |= !ok;
        slot[n] = (ok ? slot[n] : 0u) * p.stride;
    }
}
// Rows of K (or V) of one (batch, kv head); `fresh` is the chunk's own K (or
// V) when the launch also writes it to the cache (mapped only), else null.
template <bool MAPPED>
__device__ __forceinline__ Rows kv_rows(const RunArgs& a, const Ctx& c, const void* t, const void* fresh, int D,
                                        int el) {
    const uint32_t stride = static_cast<uint32_t>(a.n_kv_heads * D * el);
    if (MAPPED)
        return {static_cast<const char*>(t) + static_cast<size_t>(c.hkv) * D * el, stride,
                a.kv_map + static_cast<size_t>(c.b) * a.map_stride, a.n_slots, a.status,
                fresh ? static_cast<const char*>(fresh) + kv_index(a, c, 0, D) * el : nullptr, c.kshift};
    return {static_cast<const char*>(t) + kv_index(a, c, 0, D) * el, stride, nullptr, 0, nullptr, nullptr, 0};
}
__device__ __forceinline__ Rows q_rows(const RunArgs& a, const Ctx& c, const void* t, int D, int el) {
    return {static_cast<const char*>(t) + q_index(a, c, 0, D) * el, static_cast<uint32_t>(a.n_heads * D * el),
            nullptr, 0, nullptr};
}

// Split-K partial results: unnormalised O of row r and split s at
// ws[(r * n_split + s) * D], its (running max, sum) pair after all the O parts.
__device__ __forceinline__ float* split_o(const RunArgs& a, size_t row, int split, int D) {
    return a.ws + (row * a.n_split + split) * D;
}
__device__ __forceinline__ float2* split_ml(const RunArgs& a, size_t row, int split, int D) {
    const size_t rows = static_cast<size_t>(a.batch) * a.seq_len * a.n_heads;
    return reinterpret_cast<float2*>(a.ws + rows * a.n_split * D) + row * a.n_split + split;
}

// The chunk's own K/V rows of one query block written to their cache slots
// (the launch reads them from the chunk's tensors, so no key of this launch
// reads a slot written here while the map is one-to-one over the keys):
// by the workgroups of the first split and of the first query head of each
// kv head, each writing the tokens of its own query rows.  A slot outside
// [0, n_slots) is skipped and sets the status word.  Every load is issued
// before the first store (the compiler cannot move a load above a store
// that may alias it), so the copy costs one memory round trip, not one per
// 16-byte piece a thread moves.
template <int D, int BM, int NT>
__device__ __forceinline__ void store_chunk_rows(const RunArgs& a, const Ctx& c) {
    if (c.split != 0 || c.hq % (a.n_heads / a.n_kv_heads) != 0) return;
    constexpr int kCh = D * 2 / 16;  // 16-byte pieces of a 2-byte-element row
    constexpr int kPer = (BM * kCh + NT - 1) / NT;
    const int n = min(BM, c.S - c.q0) * kCh;
    const int32_t* map = a.kv_map + static_cast<size_t>(c.b) * a.map_stride + c.off;
    // The pieces in vector registers (arrays of them were placed in scratch
    // and LDS memory before the loops were unrolled).
    typedef uint32_t Pieces __attribute__((ext_vector_type(4 * kPer)));
    typedef int Slots __attribute__((ext_vector_type(kPer)));
    Pieces kx, vx;
    Slots slot;
#pragma unroll
    for (int p = 0; p < kPer; ++p) {  // surplus pieces re-read the last one (n >= 1)
        const int idx = min(static_cast<int>(threadIdx.x) + NT * p, n - 1);
        const int i = c.q0 + idx / kCh, ch = idx % kCh;
        const size_t src = kv_index(a, c, i, D) * 2 + 16 * ch;
        slot[p] = map[i];
        const uint4 kw = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_new) + src);
        const uint4 vw = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_new) + src);
        kx[4 * p] = kw.x, kx[4 * p + 1] = kw.y, kx[4 * p + 2] = kw.z, kx[4 * p + 3] = kw.w;
        vx[4 * p] = vw.x, vx[4 * p + 1] = vw.y, vx[4 * p + 2] = vw.z, vx[4 * p + 3] = vw.w;
    }
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
        const int idx = static_cast<int>(threadIdx.x) + NT * p;
        if (idx >= n) continue;
        const int ch = idx % kCh;
        if (static_cast<unsigned>(slot[p]) >= static_cast<unsigned>(a.n_slots)) {
            if (ch == 0) atomicOr(a.status, 1);
            continue;
        }
        const size_t dst = (static_cast<size_t>(slot[p]) * a.n_kv_heads + c.hkv) * D * 2 + 16 * ch;
        *reinterpret_cast<uint4*>(static_cast<char*>(const_cast<void*>(a.k)) + dst) =
            make_uint4(kx[4 * p], kx[4 * p + 1], kx[4 * p + 2], kx[4 * p + 3]);
        *reinterpret_cast<uint4*>(static_cast<char*>(const_cast<void*>(a.v)) + dst) =
            make_uint4(vx[4 * p], vx[4 * p + 1], vx[4 * p + 2], vx[4 * p + 3]);
    }
}

// Split-K variant of zero_rows: empty partials (O = 0, max = -inf, sum = 0).
template <int D, int BM, int NT>
__device__ void zero_partials(const RunArgs& a, const Ctx& c) {
    const int rows = min(BM, c.S - c.q0);
    for (int idx = threadIdx.x; idx < rows * (D / 4); idx += NT) {
        const int r = idx / (D / 4), col = idx % (D / 4);
        const size_t row = q_index(a, c, c.q0 + r, D) / D;
        reinterpret_cast<float4*>(split_o(a, row, c.split, D))[col] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (col == 0) *split_ml(a, row, c.split, D) = make_float2(-__builtin_huge_valf(), 0.f);
    }
    if (threadIdx.x == 0) atomicOr(a.status, 1);
}

// A batch element whose positions leave the tables: O = 0 and the status word is set.
template <int D, int BM, int NT>
__device__ void zero_rows(const RunArgs& a, const Ctx& c) {
    const int rows = min(BM, c.S - c.q0);
    for (int idx = threadIdx.x; idx < rows * (D / 4); idx += NT) {
        const int r = idx / (D / 4), col = idx % (D / 4);
        float4* dst = reinterpret_cast<float4*>(a.out + q_index(a, c, c.q0 + r, D)) + col;
        *dst = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (threadIdx.x == 0) atomicOr(a.status, 1);
}

// ------------------------------------------------ V tile: bf16 -> f16, transposed

// LDS holds V^T [D][BN + 8] f16.  Work item (kq, dc) reads keys 4kq..4kq+3 at
// dims 8dc..8dc+7; converting two keys at a time yields (key, key+1) pairs of
// one dim, i.e. the transpose for free.  Key quads are stored in the order
// 0,2,1,3 within each 16-key group so that the 8 keys one lane half feeds to
// a 16-deep MFMA step are contiguous (16-byte LDS reads).  Keys past the end
// of the sequence are clamped to the last row: they only ever meet masked
// (zero) probabilities, and a real row keeps every value finite.
template <int D, int NT>
struct VStage {
    static constexpr int kStride = BN + 8;  // f16 per V^T row
    static constexpr int kBytes = D * kStride * 2;
    static constexpr int kItems = 2 * D;    // 16 key quads x D/8 dim chunks
    static constexpr int kPer = (kItems + NT - 1) / NT;
    struct Regs {
        uint4 raw[kPer][4];
    };
    __device__ static __forceinline__ bool has(int i) { return kItems % NT == 0 || static_cast<int>(threadIdx.x % NT) + NT * i < kItems; }
    // Loads are unconditional (surplus threads re-read the last item) so that no
    // branch separates a load from its use; only the commit is guarded.
    // The key rows a thread reads: row_of(4 i + rr) for item i, key rr of its quad.
    static constexpr int kRows = 4 * kPer;
    __device__ static __forceinline__ int row_of(int n) {
        return 4 * (min(static_cast<int>(threadIdx.x % NT) + NT * (n >> 2), kItems - 1) & 15) + (n & 3);
    }
    // pre (mapped only): the rows' slot offsets read ahead (read_slots), else null.
    template <bool CLAMP, bool MAPPED>
    __device__ static __forceinline__ void load(const Rows& p, int S, int tile, Regs& r, const uint32_t* pre = nullptr) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int idx = min(static_cast<int>(threadIdx.x % NT) + NT * i, kItems - 1);
            const int kq = idx & 15, dc = idx >> 4;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                int row = 4 * kq + rr;
                if (CLAMP) row = min(row, S - 1 - tile * BN);
                r.raw[i][rr] = ld16(p.row_addr<MAPPED>(tile, row, pre ? pre + 4 * i + rr : nullptr), 16 * dc);
            }
        }
    }
    __device__ static __forceinline__ uint32_t word(const uint4& u, int i) {
        return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
    }
    __device__ static __forceinline__ void commit(const Regs& r, _Float16* lds) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            if (!has(i)) continue;
            const int idx = static_cast<int>(threadIdx.x % NT) + NT * i;
            const int kq = idx & 15, dc = idx >> 4;
            const int pos = (kq & ~3) | ((kq & 1) << 1) | ((kq >> 1) & 1);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const uint32_t w = word(r.raw[i][rr], e >> 1);
                    x[rr] = (e & 1) ? bf_hi(w) : bf_lo(w);
                }
                uint2 pk = make_uint2(pack_h2(x[0], x[1]), pack_h2(x[2], x[3]));
                *reinterpret_cast<uint2*>(lds + (8 * dc + e) * kStride + 4 * pos) = pk;
            }
        }
    }
    // O^T[db] += V^T[32db.., 16kk..] . P^T for the 16-key step kk (0..3) of the tile.
    __device__ static __forceinline__ void pv(const _Float16* lds, int kk, const f16x8& p, f32x16* o, int lq,
                                              int lh) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const f16x8 a = *reinterpret_cast<const f16x8*>(lds + (32 * db + lq) * kStride + 16 * kk + 8 * lh);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, p, o[db], 0, 0, 0);
        }
    }
};

// ------------------------------------------------ Q.K^T policy: bf16 inputs

template <int D, int NT>
struct Bf16QK {
    static constexpr int kStride = D + 8;  // f16 per K' row (16-byte pad against bank conflicts)
    static constexpr bool kSerialBlocks = false;  // the two key blocks' MFMAs may interleave
    static constexpr bool kIntScores = false;
    static constexpr int kBytes = BN * kStride * 2;
    static constexpr int kChunks = BN * D / 8;  // 16-byte chunks per K tile
    static constexpr int kPer = (kChunks + NT - 1) / NT;
    struct Q {
        f16x8 f[D / 16];
    };
    struct KRegs {
        uint4 raw[kPer];
        uint4 cs[kPer][2];  // fp32 (cos, sin) of the chunk's 4 pairs
    };
    struct KPtr {
        Rows k;
        const char* tab;  // fp32 table row of position off[b] (4 D bytes per position)
        int S;
    };
    // Q' and K' are fp16: the guard sees every converted value.
    using Guard = F16Guard;

    // Rotate 4 adjacent pairs: x' = x c - y s, y' = x s + y c; times `scale`.
    __device__ static __forceinline__ uint4 rotate8(const uint4& raw, const float4& cs0, const float4& cs1,
                                                    float scale, Guard& g) {
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        const float t[8] = {cs0.x, cs0.y, cs0.z, cs0.w, cs1.x, cs1.y, cs1.z, cs1.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float x = bf_lo(w[j]), y = bf_hi(w[j]);
            const float c = t[2 * j], s = t[2 * j + 1];
            const float xr = fmaf(x, c, -y * s), yr = fmaf(x, s, y * c);
            o[j] = pack_h2(xr * scale, yr * scale);
            g.add(o[j]);
        }
        return make_uint4(o[0], o[1], o[2], o[3]);
    }

    template <bool MAPPED>
    __device__ static __forceinline__ KPtr kptr(const RunArgs& a, const Ctx& c) {
        return {kv_rows<MAPPED>(a, c, a.k, a.k_new, D, 2),
                reinterpret_cast<const char*>(a.rope_f32 + static_cast<size_t>(c.koff) * D), c.NK};
    }

    __device__ static __forceinline__ void load_q(const RunArgs& a, const Ctx& c, int qi, float scale, Q& q,
                                                  Guard& g) {
        const int lh = (threadIdx.x & 63) >> 5;
        const bool ok = qi < c.S;
        const Rows rq = q_rows(a, c, a.q, D, 2);
        const char* tab = reinterpret_cast<const char*>(a.rope_f32 + static_cast<size_t>(c.off) * D);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const int d0 = 16 * ks + 8 * lh;
            uint4 raw = make_uint4(0, 0, 0, 0);
            float4 cs0 = make_float4(0.f, 0.f, 0.f, 0.f), cs1 = cs0;
            if (ok) {
                raw = ld16(rq.base, qi * rq.stride + 2 * d0);
                cs0 = ld16f(tab, (qi * D + d0) * 4);
                cs1 = ld16f(tab, (qi * D + d0) * 4 + 16);
            }
            q.f[ks] = __builtin_bit_cast(f16x8, rotate8(raw, cs0, cs1, scale, g));
        }
    }

    __device__ static __forceinline__ bool has(int i) { return kChunks % NT == 0 || static_cast<int>(threadIdx.x % NT) + NT * i < kChunks; }

    // The key rows a thread reads: row_of(i) for chunk i.
    static constexpr int kRows = kPer;
    __device__ static __forceinline__ int row_of(int i) {
        return min(static_cast<int>(threadIdx.x % NT) + NT * i, kChunks - 1) / (D / 8);
    }
    // CLAMP: the tile may reach past the last key (rows are clamped to it).
    // pre (mapped only): the rows' slot offsets read ahead (read_slots), else null.
    template <bool CLAMP, bool MAPPED>
    __device__ static __forceinline__ void load_k(const KPtr& p, int tile, KRegs& r, const uint32_t* pre = nullptr) {
        const char* tb = p.tab + static_cast<size_t>(tile * BN) * (D * 4);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int idx = min(static_cast<int>(threadIdx.x % NT) + NT * i, kChunks - 1);
            int row = idx / (D / 8);
            const int ch = idx % (D / 8);
            if (CLAMP) row = min(row, p.S - 1 - tile * BN);
            r.raw[i] = ld16(p.k.template row_addr<MAPPED>(tile, row, pre ? pre + i : nullptr), 16 * ch);
            r.cs[i][0] = ld16(tb, (row * D + 8 * ch) * 4);
            r.cs[i][1] = ld16(tb, (row * D + 8 * ch) * 4 + 16);
        }
    }

    // K' = RoPE(K) rounded once to fp16 (rot_pack_f32).
    __device__ static __forceinline__ uint4 rotate8_k(const uint4& raw, const uint4 (&cs)[2], Guard& g) {
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        const uint32_t t[8] = {cs[0].x, cs[0].y, cs[0].z, cs[0].w, cs[1].x, cs[1].y, cs[1].z, cs[1].w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            o[j] = rot_pack_f32(bf_lo(w[j]), bf_hi(w[j]), __uint_as_float(t[2 * j]), __uint_as_float(t[2 * j + 1]));
            g.add(o[j]);
        }
        return make_uint4(o[0], o[1], o[2], o[3]);
    }

    __device__ static __forceinline__ void commit_k(const KRegs& r, char* lds, Guard& g) {
        _Float16* kl = reinterpret_cast<_Float16*>(lds);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            if (!has(i)) continue;
            const int idx = static_cast<int>(threadIdx.x % NT) + NT * i;
            const int row = idx / (D / 8), ch = idx % (D / 8);
            *reinterpret_cast<uint4*>(kl + row * kStride + 8 * ch) = rotate8_k(r.raw[i], r.cs[i], g);
        }
    }

    // Logits (log2 units) S^T for key block kb (32 keys) of the tile x this
    // wave's 32 queries, plus `shift` (the MFMA's C operand: every lane's 16
    // entries hold minus the shift of its query).  All K' fragments of the
    // block are read from LDS before the MFMA chain is issued.
    __device__ static __forceinline__ void qk(const char* lds, int kb, const Q& q, float* s, int lq, int lh,
                                              const f32x16& shift) {
        const _Float16* row = reinterpret_cast<const _Float16*>(lds) + (32 * kb + lq) * kStride + 8 * lh;
        f16x8 a[D / 16];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) a[ks] = *reinterpret_cast<const f16x8*>(row + 16 * ks);
        f32x16 acc = shift;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[ks], q.f[ks], acc, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = acc[v];
    }
};

// ------------------------------------------------ Q.K^T policy: int16 inputs

template <int D, int NT>
struct I16QK {
    static constexpr int kRow = D + 16;  // bytes per 8-bit digit row
    // The scores of the two 32-key blocks of a tile are formed one block at a
    // time (three int32 accumulators each), which keeps the eight-wave kernels
    // within their register budget.
    static constexpr bool kSerialBlocks = true;
    static constexpr bool kIntScores = true;
    static constexpr int kPlane = BN * kRow;
    static constexpr int kBytes = 2 * kPlane;  // planes: high digit, low digit
    static constexpr int kChunks = BN * D / 8;
    static constexpr int kPer = (kChunks + NT - 1) / NT;
    struct Q {
        i32x4 h[D / 32], l[D / 32];
        float scale;
    };
    struct KRegs {
        uint4 raw[kPer];
        uint4 cs[kPer];
    };
    struct KPtr {
        Rows k;
        const char* tab;
        int S;
    };
    // The digit split is exact only for rotated values in [kDigitMin, kDigitMax].
    using Guard = DigitGuard;

    // Fixed-point rotation with round-half-up: (x C - y S + 2^13) >> 14, (x S + y C + 2^13) >> 14.
    // Every operand is an int16 value or a Q1.14 entry (|C|, |S| <= 2^14), so
    // the 24-bit multiplies (full rate) are exact: |product| <= 2^29.  Spelled
    // out because the compiler cannot see that range for the in-kernel
    // quantisation codes and falls back to the quarter-rate 32-bit multiply.
    __device__ static __forceinline__ int rot_x(int x, int y, int C, int S) {
        return (__mul24(x, C) - __mul24(y, S) + 8192) >> 14;
    }
    __device__ static __forceinline__ int rot_y(int x, int y, int C, int S) {
        return (__mul24(x, S) + __mul24(y, C) + 8192) >> 14;
    }

    // a = 128 h + l, l in [-64, 63]; returns the digit bytes h and l (both
    // int8 for a in [-16448, 16319]: at 16320, h = 128 wraps).
    __device__ static __forceinline__ void split(int a, uint32_t& h, uint32_t& l) {
        const int lo = ((a + 64) & 127) - 64;
        const int hi = (a - lo) >> 7;
        h = static_cast<uint32_t>(hi) & 0xffu;
        l = static_cast<uint32_t>(lo) & 0xffu;
    }

    // Rotate 4 pairs (one uint4 of int16) with 4 (C, S) pairs and split into digits:
    // 8 bytes per plane returned as two dwords each; the guard sees the rotated values.
    template <class G>
    __device__ static __forceinline__ void rotate_split8(const uint4& raw, const uint4& cs, uint2& h, uint2& l,
                                                         G& g) {
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        const uint32_t t[4] = {cs.x, cs.y, cs.z, cs.w};
        uint32_t hb[2] = {0, 0}, lb[2] = {0, 0};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int x = i16_lo(w[j]), y = i16_hi(w[j]);
            const int C = i16_lo(t[j]), S = i16_hi(t[j]);
            const int xr = rot_x(x, y, C, S), yr = rot_y(x, y, C, S);
            g.add(xr, yr);
            uint32_t a0, a1, b0, b1;
            split(xr, a0, a1);
            split(yr, b0, b1);
            const int sh = 16 * (j & 1);
            hb[j >> 1] |= (a0 | (b0 << 8)) << sh;
            lb[j >> 1] |= (a1 | (b1 << 8)) << sh;
        }
        h = make_uint2(hb[0], hb[1]);
        l = make_uint2(lb[0], lb[1]);
    }

    template <bool MAPPED>
    __device__ static __forceinline__ KPtr kptr(const RunArgs& a, const Ctx& c) {
        return {kv_rows<MAPPED>(a, c, a.k, a.k_new, D, 2),
                reinterpret_cast<const char*>(a.rope_q14 + static_cast<size_t>(c.koff) * D), c.NK};
    }

    __device__ static __forceinline__ void load_q(const RunArgs& a, const Ctx& c, int qi, float scale, Q& q,
                                                  Guard& g) {
        const int lh = (threadIdx.x & 63) >> 5;
        const bool ok = qi < c.S;
        const Rows rq = q_rows(a, c, a.q, D, 2);
        const char* tab = reinterpret_cast<const char*>(a.rope_q14 + static_cast<size_t>(c.off) * D);
        q.scale = scale;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const int d0 = 32 * ks + 16 * lh;
            uint2 h[2], l[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                uint4 raw = make_uint4(0, 0, 0, 0), cs = raw;
                if (ok) {
                    raw = ld16(rq.base, qi * rq.stride + 2 * (d0 + 8 * half));
                    cs = ld16(tab, (qi * D + d0 + 8 * half) * 2);
                }
                rotate_split8(raw, cs, h[half], l[half], g);
            }
            q.h[ks] = i32x4{(int)h[0].x, (int)h[0].y, (int)h[1].x, (int)h[1].y};
            q.l[ks] = i32x4{(int)l[0].x, (int)l[0].y, (int)l[1].x, (int)l[1].y};
        }
    }

    __device__ static __forceinline__ bool has(int i) { return kChunks % NT == 0 || static_cast<int>(threadIdx.x % NT) + NT * i < kChunks; }

    // The key rows a thread reads, as Bf16QK.
    static constexpr int kRows = kPer;
    __device__ static __forceinline__ int row_of(int i) {
        return min(static_cast<int>(threadIdx.x % NT) + NT * i, kChunks - 1) / (D / 8);
    }
    template <bool CLAMP, bool MAPPED>
    __device__ static __forceinline__ void load_k(const KPtr& p, int tile, KRegs& r, const uint32_t* pre = nullptr) {
        const char* tb = p.tab + static_cast<size_t>(tile * BN) * (D * 2);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int idx = min(static_cast<int>(threadIdx.x % NT) + NT * i, kChunks - 1);
            int row = idx / (D / 8);
            const int ch = idx % (D / 8);
            if (CLAMP) row = min(row, p.S - 1 - tile * BN);
            r.raw[i] = ld16(p.k.template row_addr<MAPPED>(tile, row, pre ? pre + i : nullptr), 16 * ch);
            r.cs[i] = ld16(tb, (row * D + 8 * ch) * 2);
        }
    }

    __device__ static __forceinline__ void commit_k(const KRegs& r, char* lds, Guard& g) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            if (!has(i)) continue;
            const int idx = static_cast<int>(threadIdx.x % NT) + NT * i;
            const int row = idx / (D / 8), ch = idx % (D / 8);
            uint2 h, l;
            rotate_split8(r.raw[i], r.cs[i], h, l, g);
            char* p = lds + row * kRow + 8 * ch;
            *reinterpret_cast<uint2*>(p) = h;
            *reinterpret_cast<uint2*>(p + kPlane) = l;
        }
    }

    // Exact int32 scores S^T for key block kb: 2^14 hh + 2^7 (hl + lh) + ll.
    __device__ static __forceinline__ void qk_i32(const char* lds, int kb, const Q& q, int* s, int lq, int lh) {
        const char* row = lds + (32 * kb + lq) * kRow + 16 * lh;
        i32x16 hh = {}, ll = {}, x = {};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const i32x4 ah = *reinterpret_cast<const i32x4*>(row + 32 * ks);
            const i32x4 al = *reinterpret_cast<const i32x4*>(row + kPlane + 32 * ks);
            hh = __builtin_amdgcn_mfma_i32_32x32x32_i8(ah, q.h[ks], hh, 0, 0, 0);
            ll = __builtin_amdgcn_mfma_i32_32x32x32_i8(al, q.l[ks], ll, 0, 0, 0);
            x = __builtin_amdgcn_mfma_i32_32x32x32_i8(ah, q.l[ks], x, 0, 0, 0);
            x = __builtin_amdgcn_mfma_i32_32x32x32_i8(al, q.h[ks], x, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            // (hh 2^7 + x) 2^7 + ll, the same value mod 2^32, as two shift-adds;
            // the empty asm (no instruction) keeps the compiler from spreading
            // the shifts back over three instructions
            uint32_t t = (static_cast<uint32_t>(hh[v]) << 7) + static_cast<uint32_t>(x[v]);
            asm("" : "+v"(t));
            s[v] = static_cast<int>((t << 7) + static_cast<uint32_t>(ll[v]));
        }
    }

    // Logits (log2 units) of key block kb from its int32 scores: float(score) * scale
    // plus the shift (minus the lane's shift in every entry of `shift`).
    __device__ static __forceinline__ void logits(const char*, int, const Q& q, const int* si, float* s, int,
                                                  const f32x16& shift) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = fmaf(static_cast<float>(si[v]), q.scale, shift[0]);
    }
    __device__ static __forceinline__ void qk(const char* lds, int kb, const Q& q, float* s, int lq, int lh,
                                              const f32x16& shift) {
        int si[16];
        qk_i32(lds, kb, q, si, lq, lh);
        logits(lds, kb, q, si, s, lh, shift);
    }
};

// 1/l without a divide: l = f 2^e with f in [0.5, 1), Newton-Raphson from the
// linear seed 48/17 - 32/17 f (error at most 1/17), three steps, then 2^-e.
__device__ __forceinline__ float newton_reciprocal(float l) {
    const float f = __builtin_amdgcn_frexp_mantf(l);
    const int e = __builtin_amdgcn_frexp_expf(l);
    float r = fmaf(-32.0f / 17.0f, f, 48.0f / 17.0f);
#pragma unroll
    for (int i = 0; i < 3; ++i) r = r * fmaf(-f, r, 2.0f);
    return __builtin_amdgcn_ldexpf(r, -e);
}

// ------------------------------------------------ Q.K^T policy: bf16 inputs quantised in-kernel

// Per-token dynamic int16 quantisation (the 2kiu.com retelling, §3.3): each
// (token, head) row of Q and K is scaled by 2047 / max|x| and rounded half to
// even, all in fp32, so every workgroup that stages a row derives the same
// codes; the MNN-on-K3 blog (§四) fuses the absmax scan with the quantise
// step, done here while the row is in registers.  The codes then take the
// int16 path (integer RoPE, two-digit exact int32 scores); the logit is
// s * score_scale * (m_q / 2047) * (m_k / 2047).
__device__ __forceinline__ float quant_scale(float m) { return m > 0.f ? 2047.0f / m : 0.f; }
__device__ __forceinline__ int quant_code(float x, float scale) {
    return static_cast<int>(fminf(fmaxf(__builtin_rintf(x * scale), -2048.f), 2047.f));
}
// Max over the 16 lanes of a DPP row (every lane receives it).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
    return fmaxf(x, dpp_f<0x140>(x));  // row_mirror
}

template <int D, int NT>
struct I16QuantQK : I16QK<D, NT> {
    using Base = I16QK<D, NT>;
    static constexpr int kRow = Base::kRow;
    static constexpr int kPlane = Base::kPlane;
    static constexpr int kInv = 2 * kPlane;            // 64 floats: m_k / 2047 of each key row
    static constexpr int kBytes = 2 * kPlane + BN * 4;
    static constexpr int E = D / 16;                   // elements of a key row per lane (16 lanes per row)
    static constexpr int kPasses = BN * 16 / NT;       // rows per thread per tile
    static_assert(BN * 16 % NT == 0, "whole passes");
    using Q = typename Base::Q;
    using KPtr = typename Base::KPtr;
    // Codes in [-2048, 2047] rotate to at most 2897 in magnitude: always exact.
    using Guard = NoGuard;
    struct KRegs {
        uint32_t raw[kPasses][E / 2];  // bf16 pairs
        uint32_t cs[kPasses][E / 2];   // Q1.14 (C, S) pairs
    };

    template <bool MAPPED>
    __device__ static __forceinline__ KPtr kptr(const RunArgs& a, const Ctx& c) {
        return Base::template kptr<MAPPED>(a, c);
    }

    // Q: the lane holds dims 32 ks + 16 lh .. +15 of query qi; the row max
    // comes from both lane halves.
    __device__ static __forceinline__ void load_q(const RunArgs& a, const Ctx& c, int qi, float scale, Q& q,
                                                  Guard& g) {
        const int lh = (threadIdx.x & 63) >> 5;
        const bool ok = qi < c.S;
        const Rows rq = q_rows(a, c, a.q, D, 2);
        const char* tab = reinterpret_cast<const char*>(a.rope_q14 + static_cast<size_t>(c.off) * D);
        uint4 raw[D / 32][2], cs[D / 32][2];
        float m = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int d0 = 32 * ks + 16 * lh + 8 * half;
                raw[ks][half] = ok ? ld16(rq.base, qi * rq.stride + 2 * d0) : make_uint4(0, 0, 0, 0);
                cs[ks][half] = ok ? ld16(tab, (qi * D + d0) * 2) : make_uint4(0, 0, 0, 0);
                const uint32_t w[4] = {raw[ks][half].x, raw[ks][half].y, raw[ks][half].z, raw[ks][half].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(bf_lo(w[j])), fabsf(bf_hi(w[j]))));
            }
        m = halves_max(m);
        const float qs = quant_scale(m);
        q.scale = scale * (m / 2047.0f);
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            uint2 h[2], l[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const uint32_t w[4] = {raw[ks][half].x, raw[ks][half].y, raw[ks][half].z, raw[ks][half].w};
                uint32_t cw[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    cw[j] = (static_cast<uint32_t>(quant_code(bf_lo(w[j]), qs)) & 0xffffu) |
                            (static_cast<uint32_t>(quant_code(bf_hi(w[j]), qs)) << 16);
                Base::rotate_split8(make_uint4(cw[0], cw[1], cw[2], cw[3]), cs[ks][half], h[half], l[half], g);
            }
            q.h[ks] = i32x4{(int)h[0].x, (int)h[0].y, (int)h[1].x, (int)h[1].y};
            q.l[ks] = i32x4{(int)l[0].x, (int)l[0].y, (int)l[1].x, (int)l[1].y};
        }
    }

    // K: 16 lanes per key row, lane sub holds elements [E sub, E sub + E).
    static constexpr int kRows = kPasses;
    __device__ static __forceinline__ int row_of(int i) { return static_cast<int>(threadIdx.x % NT) / 16 + (NT / 16) * i; }
    template <bool CLAMP, bool MAPPED>
    __device__ static __forceinline__ void load_k(const KPtr& p, int tile, KRegs& r, const uint32_t* pre = nullptr) {
        const int tid = threadIdx.x % NT;
        const int sub = tid & 15;
        const char* tb = p.tab + static_cast<size_t>(tile * BN) * (D * 2);
#pragma unroll
        for (int i = 0; i < kPasses; ++i) {
            int row = (tid >> 4) + (NT / 16) * i;
            if (CLAMP) row = min(row, p.S - 1 - tile * BN);
            const uint32_t* src = reinterpret_cast<const uint32_t*>(
                p.k.template row_addr<MAPPED>(tile, row, pre ? pre + i : nullptr) + 2 * E * sub);
            const uint32_t* t = reinterpret_cast<const uint32_t*>(tb + (row * D + E * sub) * 2);
#pragma unroll
            for (int e = 0; e < E / 2; ++e) {
                r.raw[i][e] = src[e];
                r.cs[i][e] = t[e];
            }
        }
    }

    __device__ static __forceinline__ void commit_k(const KRegs& r, char* lds, Guard&) {
        const int tid = threadIdx.x % NT;
        const int sub = tid & 15;
#pragma unroll
        for (int i = 0; i < kPasses; ++i) {
            const int row = (tid >> 4) + (NT / 16) * i;
            float m = 0.f;
#pragma unroll
            for (int e = 0; e < E / 2; ++e) m = fmaxf(m, fmaxf(fabsf(bf_lo(r.raw[i][e])), fabsf(bf_hi(r.raw[i][e]))));
            m = row_max16(m);
            const float ks = quant_scale(m);
            uint32_t hb[E / 4 + 1] = {}, lb[E / 4 + 1] = {};
#pragma unroll
            for (int e = 0; e < E / 2; ++e) {
                const int x = quant_code(bf_lo(r.raw[i][e]), ks), y = quant_code(bf_hi(r.raw[i][e]), ks);
                const int C = i16_lo(r.cs[i][e]), S = i16_hi(r.cs[i][e]);
                uint32_t a0, a1, b0, b1;
                Base::split(Base::rot_x(x, y, C, S), a0, a1);
                Base::split(Base::rot_y(x, y, C, S), b0, b1);
                const int sh = 16 * (e & 1);
                hb[e >> 1] |= (a0 | (b0 << 8)) << sh;
                lb[e >> 1] |= (a1 | (b1 << 8)) << sh;
            }
            char* pr = lds + row * kRow + E * sub;
#pragma unroll
            for (int pl = 0; pl < 2; ++pl) {
                const uint32_t* w = pl == 0 ? hb : lb;
                char* dst = pr + pl * kPlane;
                if (E == 8) {
                    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
                } else if (E == 4) {
                    *reinterpret_cast<uint32_t*>(dst) = w[0];
                } else {  // E == 6: six bytes at a 2-byte aligned offset
                    *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(w[0]);
                    *reinterpret_cast<uint16_t*>(dst + 2) = static_cast<uint16_t>(w[0] >> 16);
                    *reinterpret_cast<uint16_t*>(dst + 4) = static_cast<uint16_t>(w[1]);
                }
            }
            if (sub == 0) reinterpret_cast<float*>(lds + kInv)[row] = m / 2047.0f;
        }
    }

    // Logits (log2 units) from the int32 scores: float(score) * scale_q * m_k / 2047 of each key.
    __device__ static __forceinline__ void qk(const char* lds, int kb, const Q& q, float* s, int lq, int lh,
                                              const f32x16& shift) {
        int si[16];
        Base::qk_i32(lds, kb, q, si, lq, lh);
        logits(lds, kb, q, si, s, lh, shift);
    }
    __device__ static __forceinline__ void logits(const char* lds, int kb, const Q& q, const int* si, float* s,
                                                  int lh, const f32x16& shift) {
        const float* inv = reinterpret_cast<const float*>(lds + kInv) + 32 * kb + 4 * lh;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 f = *reinterpret_cast<const float4*>(inv + 8 * g);
            s[4 * g + 0] = fmaf(static_cast<float>(si[4 * g + 0]) * q.scale, f.x, shift[0]);
            s[4 * g + 1] = fmaf(static_cast<float>(si[4 * g + 1]) * q.scale, f.y, shift[0]);
            s[4 * g + 2] = fmaf(static_cast<float>(si[4 * g + 2]) * q.scale, f.z, shift[0]);
            s[4 * g + 3] = fmaf(static_cast<float>(si[4 * g + 3]) * q.scale, f.w, shift[0]);
        }
    }
};

// ------------------------------------------------ balanced staging for 8 waves

// With 512 threads every thread stages the same amount of a 64-key tile, so
// no wave waits at the tile barrier for another wave's extra staging work:
//  * K: thread (row r = tid/8, segment g = tid%8) rotates elements
//    [g D/8, (g+1) D/8) of key row r, in granules of 4 elements (2 pairs);
//  * V: thread (pair kp = tid%32, group dg = tid/32) converts dims
//    [dg D/16, (dg+1) D/16) of keys 2kp and 2kp+1; each dim gives one
//    (key, key+1) f16 pair of V^T.
// The LDS layouts are those of Bf16QK (K' rows) and VStage (V^T rows, key
// quads in the order 0,2,1,3 of each 16-key group).
template <int D, int NT>
struct Bf16Stage8 : Bf16QK<D, NT> {
    static_assert(NT == 512, "one K unit per thread needs 512 threads");
    using Base = Bf16QK<D, NT>;
    using typename Base::KPtr;
    static constexpr int kGran = D / 32;  // granules of 4 elements per thread
    struct KRegs {
        uint2 raw[kGran];
        uint4 cs[kGran];  // fp32 (cos, sin) of the granule's 2 pairs
    };
    static constexpr int kRows = 1;  // the key row a thread reads
    __device__ static __forceinline__ int row_of(int) { return static_cast<int>(threadIdx.x % NT) >> 3; }
    template <bool CLAMP, bool MAPPED>
    __device__ static __forceinline__ void load_k(const KPtr& p, int tile, KRegs& r, const uint32_t* pre = nullptr) {
        const int tid = threadIdx.x % NT;
        int row = tid >> 3;
        const int e0 = (tid & 7) * (D / 8);
        if (CLAMP) row = min(row, p.S - 1 - tile * BN);
        const char* kr = p.k.template row_addr<MAPPED>(tile, row, pre);
        const char* tb = p.tab + static_cast<size_t>(tile * BN) * (D * 4);
#pragma unroll
        for (int i = 0; i < kGran; ++i) {
            r.raw[i] = *reinterpret_cast<const uint2*>(kr + 2 * (e0 + 4 * i));
            r.cs[i] = ld16(tb, (row * D + e0 + 4 * i) * 4);
        }
    }
    __device__ static __forceinline__ void commit_k(const KRegs& r, char* lds, typename Base::Guard& g) {
        const int tid = threadIdx.x % NT;
        const int row = tid >> 3;
        const int e0 = (tid & 7) * (D / 8);
        _Float16* kl = reinterpret_cast<_Float16*>(lds) + row * Base::kStride + e0;
#pragma unroll
        for (int i = 0; i < kGran; ++i) {
            const uint32_t w[2] = {r.raw[i].x, r.raw[i].y};
            const uint32_t t[4] = {r.cs[i].x, r.cs[i].y, r.cs[i].z, r.cs[i].w};
            uint32_t o[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                o[j] = rot_pack_f32(bf_lo(w[j]), bf_hi(w[j]), __uint_as_float(t[2 * j]),
                                    __uint_as_float(t[2 * j + 1]));
                g.add(o[j]);
            }
            *reinterpret_cast<uint2*>(kl + 4 * i) = make_uint2(o[0], o[1]);
        }
    }
};

template <int D, int NT>
struct VStage8 : VStage<D, NT> {
    static_assert(NT == 512, "one V unit per thread needs 512 threads");
    using Base = VStage<D, NT>;
    static constexpr int kDims = D / 16;   // dims per thread
    static constexpr int kWords = D / 32;  // dwords per key
    struct Regs {
        uint32_t w[2][kWords];
    };
    static constexpr int kRows = 2;  // the key rows a thread reads: keys 2 kp and 2 kp + 1
    __device__ static __forceinline__ int row_of(int kk) { return 2 * (static_cast<int>(threadIdx.x % NT) & 31) + kk; }
    template <bool CLAMP, bool MAPPED>
    __device__ static __forceinline__ void load(const Rows& p, int S, int tile, Regs& r, const uint32_t* pre = nullptr) {
        const int tid = threadIdx.x % NT;
        const int kp = tid & 31, dg = tid >> 5;

#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            int row = 2 * kp + kk;
            if (CLAMP) row = min(row, S - 1 - tile * BN);
            const uint32_t* src = reinterpret_cast<const uint32_t*>(
                p.row_addr<MAPPED>(tile, row, pre ? pre + kk : nullptr) + 2 * kDims * dg);
#pragma unroll
            for (int i = 0; i < kWords; ++i) r.w[kk][i] = src[i];
        }
    }
    __device__ static __forceinline__ void commit(const Regs& r, _Float16* lds) {
        const int tid = threadIdx.x % NT;
        const int kp = tid & 31, dg = tid >> 5;
        const int q = kp >> 1;  // key quad of keys 2kp, 2kp+1
        const int pos = 4 * ((q & ~3) | ((q & 1) << 1) | ((q >> 1) & 1)) + 2 * (kp & 1);
#pragma unroll
        for (int e = 0; e < kDims; ++e) {
            const uint32_t w0 = r.w[0][e >> 1], w1 = r.w[1][e >> 1];
            const float x0 = (e & 1) ? bf_hi(w0) : bf_lo(w0);
            const float x1 = (e & 1) ? bf_hi(w1) : bf_lo(w1);
            *reinterpret_cast<uint32_t*>(lds + (kDims * dg + e) * Base::kStride + pos) = pack_h2(x0, x1);
        }
    }
};

// ------------------------------------------------ fused kernel (f16 P.V)

// One workgroup = NW waves x 32 query rows of one (batch, head).  Software
// pipeline per 64-key tile t (LDS K' double buffer holds tiles t+1 / t+2,
// V double buffer tiles t / t+1):
//   issue global loads of K(t+2), V(t+1)
//   softmax of S(t)                      (VALU, exp2)
//   S(t+1) = K'(t+1) Q'^T                (MFMA, independent of the softmax)
//   O^T += V^T(t) P~(t)^T                (MFMA)
//   rotate K(t+2) -> LDS, convert V(t+1) -> LDS
//   barrier
// so the matrix cores have independent work queued while the vector unit
// runs the softmax and the staging.  Tiles every query of the workgroup sees
// in full run a branch-free copy of the step (no masks, no clamps).
// MAPPED: cached prefill, keys read through the index map (see Ctx).
// SPLIT: the workgroup runs only its share of the key tiles and writes an
// unnormalised partial (O, running max, sum) for a merge kernel.
// PWL: the piecewise-linear softmax (see softmax_pwl): a first pass over the
// key tiles finds each row's maximum logit, the main loop then weights every
// key by the chord approximation of exp relative to that maximum.
// PP: the two-group schedule of run_pp (eight waves, three LDS buffers).
// PAIR: one barrier per two tiles (four LDS buffers each for K' and V^T, K
// staged three tiles ahead and V two): a buffer is rewritten only after the
// barrier that follows its last read, and a tile is whole one barrier before
// it is read.
//
// DBG (int16 score paths, plain launches): the kernel also stores every
// int32 score it forms for a key at or before its query to a.dbg_scores
// [B][Hq][S][S], and stores no O; V may then be any readable tensor of K's
// shape (its values do not reach the scores).
template <int D, template <int, int> class QKT, template <int, int> class VST, int NW, bool MAPPED, bool SPLIT,
          bool PWL = false, bool PP = false, bool PAIR = false, int GP = 1, bool DBG = false>
struct FusedAttn {
    static constexpr int NT = 64 * NW;
    static constexpr int BMW = 32 * NW;
    // GP > 1 packs GP query heads that share a KV head into one workgroup:
    // waves [g NW/GP, (g+1) NW/GP) take head g of the pack, each group of
    // waves the same query positions, so a K/V tile staged once serves all GP
    // heads and a block spans BMP = BMW / GP query positions.
    static_assert(GP == 1 || ((GP == 2 || GP == 4) && NW == 8), "head packing needs eight waves");
    static constexpr int BMP = BMW / GP;
    static constexpr int WPH = NW / GP;  // waves per head
    using P = QKT<D, NT>;
    using V = VST<D, NT>;
    static_assert(!PP || (NW == 8 && !PWL), "the two-group schedule needs eight waves");
    static_assert(!(PP && PAIR), "one schedule at a time");
    static constexpr int kBufs = PP ? 3 : (PAIR ? 4 : 2);
    static constexpr int KA = PAIR ? 3 : 2;  // K staged KA tiles ahead of the softmax tile
    static constexpr int VA = PAIR ? 2 : 1;  // V staged VA tiles ahead
    static constexpr int kLds = kBufs * (P::kBytes + V::kBytes);

    char* lds;
    const float* knots;  // PWL only: e^-n, n = 0..8
    Ctx c;
    int lq, lh, qw0, kq0, t_lo, n_tiles;  // kq0: the wave's first query in key space; [t_lo, n_tiles): tile range
    typename P::KPtr kp;
    Rows vp;
    typename P::KRegs kr;
    typename V::Regs vr;
    // Mapped: the slot offsets of this thread's rows of the next K and V tiles
    // to stage, read one step before their loads so that a load does not wait
    // for its map entry (without them every step waited for the map reads
    // before its tile loads: the cached launches ran 20-60% slower than plain
    // ones).  They take P::kRows + V::kRows registers.
    static constexpr bool kAhead = MAPPED;
    uint32_t km[kAhead ? P::kRows : 1], vm[kAhead ? V::kRows : 1];
    bool slot_bad;  // a slot read ahead was outside the cache (reported by finish)
    __device__ __forceinline__ void read_k_slots(int tile) {
        if constexpr (kAhead) read_slots(kp.k, c.NK, tile, km, [](int n) { return P::row_of(n); });
    }
    __device__ __forceinline__ void read_v_slots(int tile) {
        if constexpr (kAhead) read_slots(vp, c.NK, tile, vm, [](int n) { return V::row_of(n); });
    }
    // Loads of the next K / V tile in the pipeline (tile = the previous one + 1),
    // then the map entries of the tile after it.
    template <bool CLAMP>
    __device__ __forceinline__ void next_k(int tile) {
        if constexpr (kAhead) slot_offsets(kp.k, km, slot_bad);
        P::template load_k<CLAMP, MAPPED>(kp, tile, kr, kAhead ? km : nullptr);
        read_k_slots(tile + 1);
    }
    template <bool CLAMP>
    __device__ __forceinline__ void next_v(int tile) {
        if constexpr (kAhead) slot_offsets(vp, vm, slot_bad);
        V::template load<CLAMP, MAPPED>(vp, c.NK, tile, vr, kAhead ? vm : nullptr);
        read_v_slots(tile + 1);
    }
    typename P::Q q;
    typename P::Guard guard;  // range of this thread's converted Q' / K' values
    f32x16 o[D / 32];
    float m_run, l_a, l_b;
    // The scores arrive shifted by b_run, subtracted by the Q.K^T products
    // themselves (the C operand of the fp16 matrix-core path, the scaling FMA
    // of the integer ones), so the softmax exponentiates them as they are
    // instead of subtracting the running max from each.  b_run is 0 until the
    // lane's first maximum is known, then m_run, which moves only when a
    // tile's maximum passes it by more than the slack.  The shift rounds
    // differently from a later subtraction, and every launch shape of every
    // input type takes it the same way, so chunked, cached, packed and plain
    // launches give the same bits.  fp16 path: at head_dim 128 the 16 entries
    // of -b_run stay in registers, which every schedule there has to spare;
    // at 64 and 96 they would spill (the paired eight-wave 96, the
    // two-workgroup four-wave 64), so there the entries are written afresh
    // before each product (a few register moves per 32-key block, against 32
    // subtractions per tile).  The integer paths use one entry, in the FMA.
    static constexpr bool kShift = true;
    static constexpr bool kKeepShift = D == 128 && !P::kIntScores;
    float b_run;
    f32x16 nbias;  // kKeepShift: -b_run in every entry
    __device__ __forceinline__ void set_shift(float b) {
        b_run = kShift ? b : 0.f;
        if constexpr (kKeepShift) {
#pragma unroll
            for (int v = 0; v < 16; ++v) nbias[v] = -b_run;
        }
    }
    __device__ __forceinline__ f32x16 score_shift() const {
        if constexpr (kKeepShift) return nbias;
        f32x16 r = {};
        if constexpr (kShift) {
#pragma unroll
            for (int v = 0; v < 16; ++v) r[v] = -b_run;
        }
        return r;
    }
    // exp2 argument of a (shifted) score
    __device__ __forceinline__ float exp_arg(float x) const { return kShift ? x : x - m_run; }

    __device__ __forceinline__ int slot(int t) const { return PP ? (t - t_lo) % 3 : PAIR ? ((t - t_lo) & 3) : (t & 1); }
    __device__ __forceinline__ char* kbuf(int t) const { return lds + slot(t) * P::kBytes; }
    __device__ __forceinline__ _Float16* vbuf(int t) const {
        return reinterpret_cast<_Float16*>(lds + kBufs * P::kBytes + slot(t) * V::kBytes);
    }
    // Active 32-key blocks of tile t for this wave (a prefix of {0, 1}); wave-uniform.
    __device__ __forceinline__ int nact(int t) const {
        if (qw0 >= c.S) return 0;
        const int kt0 = t * BN;
        return kt0 + 32 <= kq0 + 31 ? 2 : (kt0 <= kq0 + 31 ? 1 : 0);
    }

    // Two sequential guards (not if / else-if), so the compiler cannot merge
    // the two blocks' stores through a pointer select that would push the
    // score array out of registers.
    template <bool FULL>
    __device__ __forceinline__ void qk_tile(int t, float* s) const {
        const int na = FULL ? 2 : nact(t);
        if constexpr (DBG) {
            if (na >= 1) qk_store(t, 0, s);
            if (na == 2) qk_store(t, 1, s + 16);
        } else {
            if (na >= 1) P::qk(kbuf(t), 0, q, s, lq, lh, score_shift());
            if (P::kSerialBlocks) __builtin_amdgcn_sched_barrier(0);
            if (na == 2) P::qk(kbuf(t), 1, q, s + 16, lq, lh, score_shift());
        }
    }
    // DBG: the int32 scores of key block kb, stored for keys at or before the
    // lane's query, then turned into logits as P::qk does.
    __device__ __forceinline__ void qk_store(int t, int kb, float* s) const {
        int si[16];
        P::qk_i32(kbuf(t), kb, q, si, lq, lh);
        const int qi = qw0 + lq;
        if (qi < c.S) {
            int32_t* row = a_dbg + ((static_cast<size_t>(c.b) * n_heads_dbg + c.hq) * c.S + qi) * c.S;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int key = t * BN + 32 * kb + acc_row(v, lh);
                if (key <= qi) row[key] = si[v];
            }
        }
        P::logits(kbuf(t), kb, q, si, s, lh, score_shift());
    }
    int32_t* a_dbg = nullptr;  // DBG: the score matrix, and the query head count of its layout
    int n_heads_dbg = 0;

    template <bool FULL>
    __device__ __forceinline__ void softmax(int t, int na, float* s, uint32_t* pk) {
        if (!FULL) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int k0 = t * BN + 32 * kb;
                if (kb < na && k0 + 31 > kq0) {
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (k0 + acc_row(v, lh) > kq0 + lq) s[16 * kb + v] = kNegInf;
                }
            }
        }
        // Row maximum; the two-group schedule reduces it as four independent
        // chains and forms the probabilities against the current running max
        // while the maximum is still being reduced, so only a step whose
        // maximum moves the running max (rare) forms them again.
        float m4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            if (kb < na) {
#pragma unroll
                for (int v = 0; v < 16; ++v) m4[PP ? (v & 3) : 0] = fmaxf(m4[PP ? (v & 3) : 0], s[16 * kb + v]);
            }
        if (PP) exp_tile(na, s, pk);
        // the tile's maximum, in the scores' shifted frame
        const float mx = halves_max(PP ? fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])) : m4[0]);
        const bool moved = __builtin_amdgcn_ballot_w64(mx + b_run > m_run + kRescaleSlack) != 0;
        if (moved) {
            const float m_new = fmaxf(m_run, mx + b_run);
            const float alpha = fast_exp2(m_run - m_new);
            m_run = m_new;
            l_a *= alpha;
            l_b *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
            // re-shift this tile's scores and the next tiles' products to the new max
            if (kShift && m_new != kNegInf) {
                const float d = m_new - b_run;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    if (kb < na) {
#pragma unroll
                        for (int v = 0; v < 16; ++v) s[16 * kb + v] -= d;
                    }
                set_shift(m_new);
            }
        }
        if (PP && moved) exp_tile(na, s, pk);
        const f16x2 ones = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            if (kb < na) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (!PP)
                        pk[8 * kb + j] = pack_h2(fast_exp2(exp_arg(s[16 * kb + 2 * j])),
                                                 fast_exp2(exp_arg(s[16 * kb + 2 * j + 1])));
                    const f16x2 p = __builtin_bit_cast(f16x2, pk[8 * kb + j]);
                    if (j & 1)
                        l_b = __builtin_amdgcn_fdot2(p, ones, l_b, false);
                    else
                        l_a = __builtin_amdgcn_fdot2(p, ones, l_a, false);
                }
            }
    }

    // P~ = exp2(S - m_run) as packed f16 pairs.
    __device__ __forceinline__ void exp_tile(int na, const float* s, uint32_t* pk) const {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            if (kb < na) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    pk[8 * kb + j] = pack_h2(fast_exp2(exp_arg(s[16 * kb + 2 * j])),
                                             fast_exp2(exp_arg(s[16 * kb + 2 * j + 1])));
            }
    }

    // exp(x) for x = logit - row max <= 0 as the chord of e^x between the
    // integer knots floor(x) and floor(x) + 1 (16 unit segments on [-8, 8) in
    // the 2kiu.com retelling, §3.3; only [-8, 0] occurs here), 0 below -8.
    // knots[n] = e^-n, n = 0..8, staged in LDS.
    __device__ __forceinline__ float pwl_exp(float x) const {
        if (!(x >= -8.0f)) return 0.0f;
        const float k = __builtin_floorf(x);
        const float ek = knots[min(static_cast<int>(-k), 8)];
        return ek * fmaf(1.71828182845904524f, x - k, 1.0f);
    }

    // Masked maximum of the visible logits of tile t for this lane's query.
    __device__ __forceinline__ float tile_max(int t, int na, float* s) const {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int k0 = t * BN + 32 * kb;
            if (kb < na) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const bool vis = k0 + acc_row(v, lh) <= kq0 + lq;
                    mx = fmaxf(mx, vis ? s[16 * kb + v] : kNegInf);
                }
            }
        }
        return mx;
    }

    // Weights of tile t against the fixed row maximum m_run (no rescale).
    template <bool FULL>
    __device__ __forceinline__ void softmax_pwl(int t, int na, float* s, uint32_t* pk) {
        const f16x2 ones = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            if (kb < na) {
                const int k0 = t * BN + 32 * kb;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    float w[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int v = 2 * j + e;
                        const bool vis = FULL || k0 + acc_row(v, lh) <= kq0 + lq;
                        w[e] = vis ? pwl_exp(s[16 * kb + v] + b_run - m_run) : 0.0f;
                    }
                    const uint32_t p = pack_h2(w[0], w[1]);
                    pk[8 * kb + j] = p;
                    if (j & 1)
                        l_b = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p), ones, l_b, false);
                    else
                        l_a = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p), ones, l_a, false);
                }
            }
    }

    __device__ __forceinline__ void pv_tile(int t, int na, const uint32_t* pk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            if (kb < na) {
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
                    const u32x4 b4 = {pk[8 * kb + 4 * k2], pk[8 * kb + 4 * k2 + 1], pk[8 * kb + 4 * k2 + 2],
                                      pk[8 * kb + 4 * k2 + 3]};
                    V::pv(vbuf(t), 2 * kb + k2, __builtin_bit_cast(f16x8, b4), o, lq, lh);
                }
            }
    }

    // One pipeline step for tile t; s holds S(t) on entry, sn receives S(t+1).
    // bar: end with a workgroup barrier (always, unless PAIR).
    template <bool STEADY>
    __device__ __forceinline__ void step(int t, float* s, float* sn, bool bar = true) {
        const bool ld_k = STEADY || t + KA < n_tiles;
        const bool ld_v = STEADY || t + VA < n_tiles;
        if (ld_k) next_k<!STEADY>(t + KA);
        if (ld_v) next_v<!STEADY>(t + VA);
        const int na = STEADY ? 2 : nact(t);
        uint32_t pk[16];
        if (na > 0) {
            if (PWL)
                softmax_pwl<STEADY>(t, na, s, pk);
            else
                softmax<STEADY>(t, na, s, pk);
        }
        if (STEADY || t + 1 < n_tiles) qk_tile<STEADY>(t + 1, sn);
        if (na > 0) pv_tile(t, na, pk);
        if (ld_k) P::commit_k(kr, kbuf(t + KA), guard);
        if (ld_v) V::commit(vr, vbuf(t + VA));
        if (!PAIR || bar) __syncthreads();
    }

    // Split-K: the workgroup's n_all key tiles are cut into as many equal
    // ranges of at least kMinSplitTiles tiles as the launch's split count
    // allows; this split's range is [t_lo, n_tiles), empty past that count.
    // A short prefix thus runs on few splits and writes few partials.
    __device__ __forceinline__ void split_range(const RunArgs& a, int n_all) {
        const int eff = max(1, min(a.n_split, n_all / kMinSplitTiles));
        const int per = (n_all + eff - 1) / eff;
        t_lo = min(c.split * per, n_all);
        n_tiles = min(t_lo + per, n_all);
    }
    // The partial of a row that saw no key: (max, sum) = (-inf, 0); its O part
    // is not written (the merge reads O only for a finite max).
    __device__ __forceinline__ void empty_partials(const RunArgs& a) const {
        const int qi = qw0 + lq;
        if (qi < c.S && lh == 0)
            *split_ml(a, q_index(a, c, qi, D) / D, c.split, D) = make_float2(kNegInf, 0.f);
    }

    // Two-group schedule (eight waves).  Each tile t is split into two phases
    // separated by workgroup barriers:
    //   vector phase t: commit K(t+2) -> K' and V(t+1) -> V^T (registers loaded
    //                   two phases earlier), issue the global loads of K(t+3)
    //                   and V(t+2), softmax of S(t) -> P~(t)     (VALU, exp2)
    //   matrix phase t: O^T += V^T(t) P~(t)^T, S(t+1) = K'(t+1) Q'^T  (MFMA)
    // Waves 4-7 pass one extra barrier before the loop and waves 0-3 one after
    // it, so the second group runs one phase behind the first: on each SIMD one
    // wave feeds the matrix cores while the other keeps the vector unit busy,
    // and S needs one register buffer instead of two.  Three LDS buffers for K'
    // and V^T keep every tile whole from the end of the phase that completes it
    // until the lagging group has read it.
    // A workgroup barrier that the compiler may not move any instruction
    // across, so each phase keeps its own work.
    __device__ __forceinline__ static void phase_barrier() {
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    }
    template <bool STEADY>
    __device__ __forceinline__ int vector_phase(int t, float* s, uint32_t* pk) {
        if (STEADY || t + 2 < n_tiles) P::commit_k(kr, kbuf(t + 2), guard);
        if (STEADY || t + 1 < n_tiles) V::commit(vr, vbuf(t + 1));
        if (STEADY || t + 3 < n_tiles) next_k<!STEADY>(t + 3);
        if (STEADY || t + 2 < n_tiles) next_v<!STEADY>(t + 2);
        const int na = STEADY ? 2 : nact(t);
        if (na > 0) softmax<STEADY>(t, na, s, pk);
        return na;
    }
    template <bool STEADY>
    __device__ __forceinline__ void matrix_phase(int t, int na, const uint32_t* pk, float* s) {
        if (na > 0) pv_tile(t, na, pk);
        if (STEADY || t + 1 < n_tiles) qk_tile<STEADY>(t + 1, s);
    }

    __device__ __forceinline__ void run_pp(const RunArgs& a, float logit_scale) {
        const int lane = threadIdx.x & 63;
        const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
        lq = lane & 31;
        lh = lane >> 5;
        qw0 = c.q0 + 32 * (w % WPH);
        kq0 = c.kshift + qw0;
        const int n_all = (c.kshift + min(c.q0 + BMP, c.S) + BN - 1) / BN;
        const int n_full = min((c.kshift + c.q0) / BN, n_all);
        t_lo = 0;
        n_tiles = n_all;
        if (SPLIT) {
            split_range(a, n_all);
            if (t_lo >= n_tiles) {  // empty split (workgroup-uniform): no barrier has run yet
                empty_partials(a);
                return;
            }
        }
        kp = P::template kptr<MAPPED>(a, c);
        vp = kv_rows<MAPPED>(a, c, a.v, a.v_new, D, 2);

        // Prologue: K'(t_lo), K'(t_lo+1) and V^T(t_lo) in LDS; K(t_lo+2) and
        // V(t_lo+1) in registers for the first vector phase.  An empty split
        // loads nothing (a clamped row past the last key would be negative).
        // All loads are issued before any commit (one memory round trip); K(t_lo+2)
        // and V(t_lo+1) stay in kr / vr for the first vector phase.
        const bool any = t_lo < n_tiles;
        typename P::KRegs kr0, kr1;
        typename V::Regs vr0;
        if (any) {
            P::template load_k<true, MAPPED>(kp, t_lo, kr0);
            V::template load<true, MAPPED>(vp, c.NK, t_lo, vr0);
        }
        if (t_lo + 1 < n_tiles) {
            P::template load_k<true, MAPPED>(kp, t_lo + 1, kr1);
            V::template load<true, MAPPED>(vp, c.NK, t_lo + 1, vr);
        }
        if (t_lo + 2 < n_tiles) P::template load_k<true, MAPPED>(kp, t_lo + 2, kr);
        slot_bad = false;
        if (any) {  // the first vector phase's K / V tiles
            read_k_slots(t_lo + 3);
            read_v_slots(t_lo + 2);
        }
        P::load_q(a, c, qw0 + lq, logit_scale, q, guard);
        if (any) {
            P::commit_k(kr0, kbuf(t_lo), guard);
            V::commit(vr0, vbuf(t_lo));
        }
        if (t_lo + 1 < n_tiles) P::commit_k(kr1, kbuf(t_lo + 1), guard);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
        m_run = kNegInf;
        set_shift(0.f);
        l_a = 0.f;
        l_b = 0.f;
        __syncthreads();
        float s[32];
        if (any) qk_tile<false>(t_lo, s);

        const bool lagging = w >= 4;  // waves w and w + 4 share a SIMD
        if (lagging) __syncthreads();
        int t = t_lo;
        const int t_steady = SPLIT ? min(n_full, n_tiles) : n_full;
        // Steady tiles load K(t+3) and V(t+2) unclamped and run an unmasked
        // softmax: t+3 must lie below n_full.
        for (; t + 3 < t_steady; ++t) {
            uint32_t pk[16];
            vector_phase<true>(t, s, pk);
            phase_barrier();
            matrix_phase<true>(t, 2, pk, s);
            phase_barrier();
        }
        for (; t < n_tiles; ++t) {
            uint32_t pk[16];
            const int na = vector_phase<false>(t, s, pk);
            phase_barrier();
            matrix_phase<false>(t, na, pk, s);
            phase_barrier();
        }
        if (!lagging) __syncthreads();
        finish(a);
    }

    // Bit 1 of the status word: a converted Q' / K' left its range (this
    // thread's guard) or a row of O (or of a partial) is not finite.
    __device__ __forceinline__ void report_range(const RunArgs& a, bool bad) const {
        if (bad) atomicOr(a.status, 2);
    }

    // Normalised O (or the split-K partial) of the wave's rows.
    __device__ __forceinline__ void finish(const RunArgs& a) {
        if (kAhead && slot_bad) atomicOr(a.status, 1);
        const bool gbad = guard.bad();
        if (DBG || qw0 >= c.S) {
            report_range(a, gbad);
            return;
        }
        if (SPLIT) {
            // A row that saw no key of this split (its first tile starts past
            // the row) keeps m_run = -inf: an empty partial.
            const float l = halves_sum(l_a + l_b);  // cross-lane: every lane takes part
            if (m_run == kNegInf) {
                report_range(a, gbad);
                empty_partials(a);
                return;
            }
            const int qi = qw0 + lq;
            bool bad = gbad || !__builtin_isfinite(l);
            if (qi < c.S) {
                const size_t row = q_index(a, c, qi, D) / D;
                float* dst = split_o(a, row, c.split, D);
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const float4 val = make_float4(o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2],
                                                       o[db][4 * g + 3]);
                        bad |= !__builtin_isfinite(val.x + val.y + val.z + val.w);
                        *reinterpret_cast<float4*>(dst + 32 * db + 8 * g + 4 * lh) = val;
                    }
                if (lh == 0) *split_ml(a, row, c.split, D) = make_float2(m_run, l);
            }
            report_range(a, bad);
            return;
        }
        const float inv = PWL ? newton_reciprocal(halves_sum(l_a + l_b)) : 1.0f / halves_sum(l_a + l_b);
        const int qi = qw0 + lq;
        bool bad = gbad;
        if (qi < c.S) {
            float* orow = a.out + q_index(a, c, qi, D);
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 val = make_float4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv,
                                                   o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
                    bad |= !__builtin_isfinite(val.x + val.y + val.z + val.w);
                    *reinterpret_cast<float4*>(orow + 32 * db + 8 * g + 4 * lh) = val;
                }
        }
        report_range(a, bad);
    }

    __device__ __forceinline__ void run(const RunArgs& a, float logit_scale) {
        const int lane = threadIdx.x & 63;
        const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
        lq = lane & 31;
        lh = lane >> 5;
        qw0 = c.q0 + 32 * (w % WPH);
        kq0 = c.kshift + qw0;
        const int n_all = (c.kshift + min(c.q0 + BMP, c.S) + BN - 1) / BN;
        const int n_full = min((c.kshift + c.q0) / BN, n_all);  // tiles every query of the workgroup sees whole
        t_lo = 0;
        n_tiles = n_all;
        if (SPLIT) {
            split_range(a, n_all);
            if (t_lo >= n_tiles) {  // empty split (workgroup-uniform): no barrier has run yet
                empty_partials(a);
                return;
            }
        }
        kp = P::template kptr<MAPPED>(a, c);
        vp = kv_rows<MAPPED>(a, c, a.v, a.v_new, D, 2);

        float pwl_max = kNegInf;
        if (PWL) {
            // First pass: the maximum visible logit of every query row.
            P::load_q(a, c, qw0 + lq, logit_scale, q, guard);
            for (int t = 0; t < n_tiles; ++t) {
                P::template load_k<true, MAPPED>(kp, t, kr);
                __syncthreads();  // the previous tile's reads are done
                P::commit_k(kr, kbuf(0), guard);
                __syncthreads();
                const int na = nact(t);
                float s1[32];
                if (na >= 1) P::qk(kbuf(0), 0, q, s1, lq, lh, f32x16{});
                if (na == 2) P::qk(kbuf(0), 1, q, s1 + 16, lq, lh, f32x16{});
                if (na > 0) pwl_max = fmaxf(pwl_max, tile_max(t, na, s1));
            }
            pwl_max = halves_max(pwl_max);
            __syncthreads();  // buffer 0 is restaged below
        }

        // An empty split (t_lo == n_all) loads no tile: a clamped row of a tile
        // past the last key would be negative, and row offsets are unsigned.
        // Every load of the first tiles (and Q's) is issued before any of them
        // is committed, so the prologue waits for one memory round trip.
        const bool any = !SPLIT || t_lo < n_tiles;
        const bool k1 = t_lo + 1 < n_tiles, v1 = PAIR && t_lo + 1 < n_tiles, k2 = PAIR && t_lo + 2 < n_tiles;
        typename P::KRegs kr1, kr2;
        typename V::Regs vr1;
        if (any) {
            P::template load_k<true, MAPPED>(kp, t_lo, kr);
            V::template load<true, MAPPED>(vp, c.NK, t_lo, vr);
        }
        if (k1) P::template load_k<true, MAPPED>(kp, t_lo + 1, kr1);
        if (v1) V::template load<true, MAPPED>(vp, c.NK, t_lo + 1, vr1);
        if (k2) P::template load_k<true, MAPPED>(kp, t_lo + 2, kr2);
        slot_bad = false;
        if (any) {  // the first step's K / V tiles
            read_k_slots(t_lo + KA);
            read_v_slots(t_lo + VA);
        }
        P::load_q(a, c, qw0 + lq, logit_scale, q, guard);
        if (any) {
            P::commit_k(kr, kbuf(t_lo), guard);
            V::commit(vr, vbuf(t_lo));
        }
        if (k1) P::commit_k(kr1, kbuf(t_lo + 1), guard);
        if (v1) V::commit(vr1, vbuf(t_lo + 1));
        if (k2) P::commit_k(kr2, kbuf(t_lo + 2), guard);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
        m_run = PWL ? pwl_max : kNegInf;
        set_shift(PWL && pwl_max != kNegInf ? pwl_max : 0.f);
        l_a = 0.f;
        l_b = 0.f;
        __syncthreads();
        float sa[32], sb[32];
        if (any) qk_tile<false>(t_lo, sa);
        __syncthreads();  // every wave has read K'(t_lo) before the first step overwrites that buffer

        // A steady pair loads K(t+2), K(t+3) and V(t+1), V(t+2) unclamped and runs
        // the softmax of tiles t, t+1 unmasked: every one of those tiles must lie
        // below n_full (tile n_full itself may reach past the last key) and in range.
        int t = t_lo;
        const int t_steady = SPLIT ? min(n_full, n_tiles) : n_full;
        // (PAIR: a steady pair stages K(t+4) and V(t+3), so t+4 lies below n_full.)
        for (; t + KA + 1 < t_steady; t += 2) {
            step<true>(t, sa, sb, false);
            step<true>(t + 1, sb, sa, true);
        }
        for (; t < n_tiles; t += 2) {
            const bool two = t + 1 < n_tiles;
            step<false>(t, sa, sb, !two);
            if (two) step<false>(t + 1, sb, sa, true);
        }

        finish(a);
    }
};

template <int D, template <int, int> class QKT, template <int, int> class VST, int NW, int MINB, bool MAPPED,
          bool SPLIT = false, bool PWL = false, bool PP = false, bool PAIR = false, int GP = 1, bool DBG = false>
__global__ __launch_bounds__(64 * NW, MINB) void attn_fwd_kernel(RunArgs a, float logit_scale) {
    using K = FusedAttn<D, QKT, VST, NW, MAPPED, SPLIT, PWL, PP, PAIR, GP, DBG>;
    __shared__ __attribute__((aligned(16))) char lds[K::kLds];
    __shared__ float knots[PWL ? 9 : 1];
    K k;
    k.lds = lds;
    k.knots = knots;
    if (DBG) {
        k.a_dbg = a.dbg_scores;
        k.n_heads_dbg = a.n_heads;
    }
    if (PWL && threadIdx.x < 9) {
        // e^-n, n = 0..8
        constexpr float kE[9] = {1.0f, 0.36787944117144233f, 0.1353352832366127f, 0.049787068367863944f,
                                 0.01831563888873418f, 0.006737946999085467f, 0.0024787521766663585f,
                                 0.0009118819655545162f, 0.00033546262790251185f};
        knots[threadIdx.x] = kE[threadIdx.x];
    }
    // One query block, or two in a paired launch (eight-wave kernels only).
    // With head packing, blocks are enumerated over (batch, head pair) and
    // each wave then moves to its own head of the pair.
    const bool paired = !SPLIT && NW == 8 && a.paired;
    const int n_qblocks = (a.seq_len + K::BMP - 1) / K::BMP;
    const int bid = SPLIT ? static_cast<int>(blockIdx.x) / a.n_split : static_cast<int>(blockIdx.x);
    const int split = SPLIT ? static_cast<int>(blockIdx.x) % a.n_split : 0;
    const int hw = GP > 1 ? __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)) / K::WPH : 0;
    auto block = [&](int item) {
        BlockPos bp = paired ? map_pair(n_qblocks, a.batch, a.n_heads / GP, bid, item)
                             : map_block(n_qblocks, a.batch, a.n_heads / GP, bid);
        bp.hq *= GP;
        return bp;
    };
    // A sequence whose positions leave the tables: every head of the block gets O = 0.
    auto zero_block = [&]() {
#pragma unroll
        for (int h = 0; h < GP; ++h) {
            Ctx cz = k.c;
            cz.hq += h;
            if (SPLIT)
                zero_partials<D, K::BMP, K::NT>(a, cz);
            else
                zero_rows<D, K::BMP, K::NT>(a, cz);
        }
    };
    const BlockPos bp = block(0);
    const bool ok = make_ctx_at<K::BMP, MAPPED>(a, bp, split, k.c);
    if (!ok) {
        if (DBG) {
            if (threadIdx.x == 0) atomicOr(a.status, 1);  // no O to zero
            return;
        }
        zero_block();
    } else {
        if (MAPPED && a.k_new) store_chunk_rows<D, K::BMP, K::NT>(a, k.c);
        k.c.hq += hw;
        if (PP)
            k.run_pp(a, logit_scale);
        else
            k.run(a, logit_scale);
    }
    if (!paired || 2 * bp.qb == n_qblocks - 1) return;  // the middle block of an odd count runs alone
    // Second block of the pair: same (batch, head), so the same validity.
    make_ctx_at<K::BMP, MAPPED>(a, block(1), split, k.c);
    if (!ok) {
        zero_block();
        return;
    }
    if (MAPPED && a.k_new) store_chunk_rows<D, K::BMP, K::NT>(a, k.c);
    k.c.hq += hw;
    __syncthreads();  // every wave is done with the first block's LDS tiles
    if (PP)
        k.run_pp(a, logit_scale);
    else
        k.run(a, logit_scale);
}

// ------------------------------------------------ fp32 kernel (fp32 matrix cores)

template <int D, bool MAPPED>
__global__ __launch_bounds__(kThreads) void attn_fwd_f32_kernel(RunArgs a, float logit_scale) {
    constexpr int kStride = D + 4;
    __shared__ __attribute__((aligned(16))) float ks_[BN * kStride];
    __shared__ __attribute__((aligned(16))) float vs_[BN * kStride];

    Ctx c;
    if (!make_ctx<BM, MAPPED>(a, c)) {
        zero_rows<D, BM, kThreads>(a, c);
        return;
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int lq = lane & 31, lh = lane >> 5;
    const int qw0 = c.q0 + 32 * w;
    const int kq0 = c.kshift + qw0;
    const int n_tiles = (c.kshift + min(c.q0 + BM, c.S) + BN - 1) / BN;
    const float* qg = static_cast<const float*>(a.q);
    const Rows kr_ = kv_rows<MAPPED>(a, c, a.k, nullptr, D, 4);
    const Rows vr_ = kv_rows<MAPPED>(a, c, a.v, nullptr, D, 4);

    // Q' of query qw0+lq: lane half lh keeps component lh of every pair (d = 2ks + lh).
    float qv[D / 2];
    {
        const int qi = qw0 + lq;
        const bool ok = qi < c.S;
#pragma unroll
        for (int k = 0; k < D / 2; ++k) {
            float x = 0.f, y = 0.f, cs = 0.f, sn = 0.f;
            if (ok) {
                const float2 xy = *reinterpret_cast<const float2*>(qg + q_index(a, c, qi, D) + 2 * k);
                const float2 t = *reinterpret_cast<const float2*>(a.rope_f32 + static_cast<size_t>(c.off + qi) * D + 2 * k);
                x = xy.x, y = xy.y, cs = t.x, sn = t.y;
            }
            qv[k] = (lh ? fmaf(x, sn, y * cs) : fmaf(x, cs, -y * sn)) * logit_scale;
        }
    }
    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    float m_run = kNegInf, l_run = 0.f;

    for (int t = 0; t < n_tiles; ++t) {
        __syncthreads();
        for (int idx = threadIdx.x; idx < BN * (D / 4); idx += kThreads) {
            const int row = idx / (D / 4), ch = idx % (D / 4);
            const int key = t * BN + row;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx, tc = kx;
            if (key < c.NK) {
                kx = ld16f(kr_.tile_base<MAPPED>(t), kr_.row_off<MAPPED>(t, row) + 16 * ch);
                vx = ld16f(vr_.tile_base<MAPPED>(t), vr_.row_off<MAPPED>(t, row) + 16 * ch);
                tc = *reinterpret_cast<const float4*>(a.rope_f32 + static_cast<size_t>(c.koff + key) * D + 4 * ch);
            }
            const float4 kr = make_float4(fmaf(kx.x, tc.x, -kx.y * tc.y), fmaf(kx.x, tc.y, kx.y * tc.x),
                                          fmaf(kx.z, tc.z, -kx.w * tc.w), fmaf(kx.z, tc.w, kx.w * tc.z));
            *reinterpret_cast<float4*>(ks_ + row * kStride + 4 * ch) = kr;
            *reinterpret_cast<float4*>(vs_ + row * kStride + 4 * ch) = vx;
        }
        __syncthreads();
        const int kt0 = t * BN;
        int nact = kt0 + 32 <= kq0 + 31 ? 2 : (kt0 <= kq0 + 31 ? 1 : 0);
        if (qw0 >= c.S) nact = 0;
        if (nact == 0) continue;
        float s[2][16];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb >= nact) break;
            f32x16 acc = {};
            const float* row = ks_ + (32 * kb + lq) * kStride + lh;
#pragma unroll
            for (int k = 0; k < D / 2; ++k) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(row[2 * k], qv[k], acc, 0, 0, 0);
            const int k0 = kt0 + 32 * kb;
#pragma unroll
            for (int v = 0; v < 16; ++v) s[kb][v] = (k0 + acc_row(v, lh) > kq0 + lq) ? kNegInf : acc[v];
        }
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            if (kb < nact) {
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
            }
        mx = halves_max(mx);
        const float m_new = fmaxf(m_run, mx);
        if (__builtin_amdgcn_ballot_w64(m_new > m_run + kRescaleSlack)) {
            const float alpha = fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb >= nact) break;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = fast_exp2(s[kb][v] - m_run);
                l_run += p;
                const float* vrow = vs_ + (32 * kb + acc_row(v, lh)) * kStride + lq;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[32 * db], p, o[db], 0, 0, 0);
            }
        }
    }

    if (qw0 >= c.S) return;
    const float inv = 1.0f / halves_sum(l_run);
    const int qi = qw0 + lq;
    if (qi < c.S) {
        float* orow = a.out + q_index(a, c, qi, D);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 val = make_float4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                                               o[db][4 * g + 3] * inv);
                *reinterpret_cast<float4*>(orow + 32 * db + 8 * g + 4 * lh) = val;
            }
    }
}

// ------------------------------------------------ KV cache update

// New token i of sequence b (logical position off[b] + i) is copied to slot
// kv_map[b][off[b] + i] of the caches; nothing else is touched.  One
// workgroup per new token: the offset and the slot are looked up once, then
// the K and V rows are copied in 16-byte chunks.  A sequence whose chunk
// leaves the map row, or a slot outside [0, n_slots), is skipped and sets the
// status word.
__global__ __launch_bounds__(kThreads) void kv_cache_update_kernel(RunArgs a, uint32_t row_bytes, char* dk,
                                                                   char* dv) {
    const uint32_t tok = blockIdx.x;  // < batch * seq_len (checked at launch)
    const int b = static_cast<int>(tok / static_cast<uint32_t>(a.seq_len));
    const int i = static_cast<int>(tok - static_cast<uint32_t>(b) * static_cast<uint32_t>(a.seq_len));
    const int off = a.pos_offsets ? a.pos_offsets[b] : 0;
    if (off < 0 || static_cast<long long>(off) + a.seq_len > a.map_stride) {
        if (threadIdx.x == 0) atomicOr(a.status, 1);
        return;
    }
    const int slot = a.kv_map[static_cast<size_t>(b) * a.map_stride + off + i];
    if (static_cast<unsigned>(slot) >= static_cast<unsigned>(a.n_slots)) {
        if (threadIdx.x == 0) atomicOr(a.status, 1);
        return;
    }
    const char* ks = static_cast<const char*>(a.k) + static_cast<size_t>(tok) * row_bytes;
    const char* vs = static_cast<const char*>(a.v) + static_cast<size_t>(tok) * row_bytes;
    char* kd = dk + static_cast<size_t>(slot) * row_bytes;
    char* vd = dv + static_cast<size_t>(slot) * row_bytes;
    for (uint32_t c = 16u * threadIdx.x; c < row_bytes; c += 16u * kThreads) {
        const uint4 kx = *reinterpret_cast<const uint4*>(ks + c);
        const uint4 vx = *reinterpret_cast<const uint4*>(vs + c);
        *reinterpret_cast<uint4*>(kd + c) = kx;
        *reinterpret_cast<uint4*>(vd + c) = vx;
    }
}

// ------------------------------------------------ int16 test kernels

// RoPE of int16 rows through the int16 path's own K staging: a workgroup of
// NT threads (the NT of the prefill launch of this shape) loads one 64-row tile
// of one (batch, head) with its Q1.14 table rows (load_k), rotates it and
// splits it into the two digit planes in LDS (commit_k, rotate_split8), and
// writes back x' = 128 h + l read from the planes.  a.k is the input,
// a.n_kv_heads its head count.
template <int D, int NT>
__global__ __launch_bounds__(NT) void debug_rope_i16_kernel(RunArgs a, int16_t* dst) {
    using P = I16QK<D, NT>;
    __shared__ __attribute__((aligned(16))) char lds[P::kBytes];
    const int n_tiles = (a.seq_len + BN - 1) / BN;
    const int tile = static_cast<int>(blockIdx.x) % n_tiles;
    const int bh = static_cast<int>(blockIdx.x) / n_tiles;
    Ctx c;
    c.b = bh / a.n_kv_heads;
    c.hkv = bh % a.n_kv_heads;
    c.hq = c.hkv;
    c.S = a.seq_len;
    c.q0 = 0;
    c.off = a.pos_offsets ? a.pos_offsets[c.b] : 0;
    c.koff = c.off;
    c.kshift = 0;
    c.NK = c.S;
    c.split = 0;
    const int rows = min(BN, c.S - tile * BN);
    int16_t* out = dst + kv_index(a, c, tile * BN, D);
    const uint32_t stride = static_cast<uint32_t>(a.n_kv_heads) * D;
    if (c.off < 0 || static_cast<long long>(c.off) + c.S > a.max_seq) {
        for (int idx = threadIdx.x; idx < rows * D; idx += NT) out[(idx / D) * stride + idx % D] = 0;
        if (threadIdx.x == 0) atomicOr(a.status, 1);
        return;
    }
    const typename P::KPtr kp = P::template kptr<false>(a, c);
    typename P::KRegs kr;
    typename P::Guard g;
    P::template load_k<true, false>(kp, tile, kr);
    P::commit_k(kr, lds, g);
    __syncthreads();
    for (int idx = threadIdx.x; idx < rows * D; idx += NT) {
        const int r = idx / D, d = idx % D;
        const int h = static_cast<int8_t>(lds[r * P::kRow + d]);
        const int l = static_cast<int8_t>(lds[P::kPlane + r * P::kRow + d]);
        out[r * stride + d] = static_cast<int16_t>(128 * h + l);
    }
    if (g.bad()) atomicOr(a.status, 2);
}

// ------------------------------------------------ launch helpers

dim3 grid_for(const RunArgs& a, int bm) {
    const int n_qblocks = (a.seq_len + bm - 1) / bm;
    return dim3(static_cast<unsigned>(n_qblocks) * a.batch * a.n_heads);
}

}  // namespace

// Compute units of the current device (cached per device).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Pairs of query blocks (n-1-j, j) all cover the same number of key tiles, so
// a paired launch balances exactly when its pairs fill whole rounds of one
// workgroup per CU.  Taken when the last round is at least 7/8 full: then
// nearly every CU would run two blocks of an unpaired launch back to back.
bool use_pairs(const RunArgs& a, int rows, int head_pack) {
    const long long n_qb = (a.seq_len + rows - 1) / rows;
    if (n_qb < 2) return false;
    const long long cus = device_cus();
    const long long pairs = (n_qb + 1) / 2 * a.batch * (a.n_heads / head_pack);
    const long long last = pairs % cus;
    return pairs >= cus * 7 / 8 && (last == 0 || last >= cus * 7 / 8);
}

namespace {

// Workgroup shape from prefill_uses_eight_waves; a non-null index map selects
// the cached-prefill instantiation, n_split > 1 (with the map) the split-K one.
template <int D, bool M, bool SP>
void launch_bf16_dm(const RunArgs& a, hipStream_t s) {
    const int ns = SP ? a.n_split : 1;
    // Launches whose query heads share KV heads in groups of 4 (or 2) pack 4
    // (2) heads of a group into one workgroup of 64 (128) query positions.
    const int group = a.n_heads / a.n_kv_heads;
    if (prefill_uses_eight_waves(a) && group % 2 == 0) {
        const int gp = group % 4 == 0 ? 4 : 2, rows = 256 / gp;
        const unsigned n_qb = static_cast<unsigned>((a.seq_len + rows - 1) / rows);
        dim3 g(n_qb * a.batch * (a.n_heads / gp) * ns);
        RunArgs b = a;
        if (!SP && use_pairs(a, rows, gp)) {
            b.paired = 1;
            g.x = (n_qb + 1) / 2 * a.batch * (a.n_heads / gp);
        }
        constexpr bool kPP = D == 128;
        if (gp == 4)
            hipLaunchKernelGGL((attn_fwd_kernel<D, Bf16Stage8, VStage8, 8, 1, M, SP, false, kPP, !kPP, 4>), g,
                               dim3(512), 0, s, b, a.score_scale * kLog2e);
        else
            hipLaunchKernelGGL((attn_fwd_kernel<D, Bf16Stage8, VStage8, 8, 1, M, SP, false, kPP, !kPP, 2>), g,
                               dim3(512), 0, s, b, a.score_scale * kLog2e);
        return;
    }
    if (prefill_uses_eight_waves(a)) {
        dim3 g = grid_for(a, 256);
        g.x *= ns;
        RunArgs b = a;
        if (!SP && use_pairs(a)) {
            b.paired = 1;
            g.x = static_cast<unsigned>(((a.seq_len + 255) / 256 + 1) / 2) * a.batch * a.n_heads;
        }
        // head_dim 128 runs the two-group schedule (its single S buffer keeps
        // the kernel out of spills, cached and split launches included), the
        // others one barrier per two tiles (split launches too: the chunked
        // long prompt ran 1% faster than with one barrier per tile).
        constexpr bool kPP = D == 128;
        hipLaunchKernelGGL((attn_fwd_kernel<D, Bf16Stage8, VStage8, 8, 1, M, SP, false, kPP, !kPP>), g,
                           dim3(512), 0, s, b, a.score_scale * kLog2e);
    } else {
        dim3 g = grid_for(a, 128);
        g.x *= ns;
        // Two workgroups per CU fit only head_dim 64 in 256 VGPRs; at 96 and 128
        // the whole-tile staging registers spilled (up to 400 bytes per lane)
        // and one workgroup per CU, with the accumulators in AGPRs, is faster.
        hipLaunchKernelGGL((attn_fwd_kernel<D, Bf16QK, VStage, 4, D == 64 ? 2 : 1, M, SP>), g, dim3(256), 0, s, a,
                           a.score_scale * kLog2e);
    }
}
template <int D>
hipError_t launch_bf16_d(const RunArgs& a, hipStream_t s) {
    if (a.kv_map && a.n_split > 1)
        launch_bf16_dm<D, true, true>(a, s);
    else if (a.kv_map)
        launch_bf16_dm<D, true, false>(a, s);
    else
        launch_bf16_dm<D, false, false>(a, s);
    return hipGetLastError();
}
// DBG: the same launch with the score-storing instantiation (plain launches only).
template <int D, template <int, int> class QKT, bool DBG = false>
hipError_t launch_int_d(const RunArgs& a, hipStream_t s) {
    // Plain head_dim 128 launches that fill the chip run the eight-wave
    // two-group kernel (half the K staging and quantisation per query row); at
    // 64 and 96 the int variants' extra Q digit planes push it into spills.
    if constexpr (D == 128) {
        if (!a.kv_map && prefill_uses_eight_waves(a)) {
            dim3 g = grid_for(a, 256);
            RunArgs b = a;
            if (use_pairs(a)) {
                b.paired = 1;
                g.x = static_cast<unsigned>(((a.seq_len + 255) / 256 + 1) / 2) * a.batch * a.n_heads;
            }
            hipLaunchKernelGGL((attn_fwd_kernel<D, QKT, VStage8, 8, 1, false, false, false, true, false, 1, DBG>), g,
                               dim3(512), 0, s, b, a.score_scale * kLog2e);
            return hipGetLastError();
        }
    }
    if constexpr (DBG) {
        if (a.kv_map) return hipErrorInvalidValue;
        hipLaunchKernelGGL((attn_fwd_kernel<D, QKT, VStage, 4, 1, false, false, false, false, false, 1, true>),
                           grid_for(a, 128), dim3(256), 0, s, a, a.score_scale * kLog2e);
        return hipGetLastError();
    }
    if (a.kv_map && a.n_split > 1) {
        dim3 g = grid_for(a, 128);
        g.x *= a.n_split;
        hipLaunchKernelGGL((attn_fwd_kernel<D, QKT, VStage, 4, 1, true, true>), g, dim3(256), 0, s, a,
                           a.score_scale * kLog2e);
    } else if (a.kv_map) {
        hipLaunchKernelGGL((attn_fwd_kernel<D, QKT, VStage, 4, 1, true>), grid_for(a, 128), dim3(256), 0, s, a,
                           a.score_scale * kLog2e);
    } else {
        hipLaunchKernelGGL((attn_fwd_kernel<D, QKT, VStage, 4, 1, false>), grid_for(a, 128), dim3(256), 0, s, a,
                           a.score_scale * kLog2e);
    }
    return hipGetLastError();
}
template <int D>
hipError_t launch_i16_d(const RunArgs& a, hipStream_t s) { return launch_int_d<D, I16QK>(a, s); }
template <int D>
hipError_t launch_i16q_d(const RunArgs& a, hipStream_t s) { return launch_int_d<D, I16QuantQK>(a, s); }
// Piecewise-linear softmax: logits in natural units (no log2 e factor).
template <int D>
hipError_t launch_i16pwl_d(const RunArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((attn_fwd_kernel<D, I16QK, VStage, 4, 1, false, false, true>), grid_for(a, 128), dim3(256), 0,
                       s, a, a.score_scale);
    return hipGetLastError();
}
template <int D>
hipError_t launch_f32_d(const RunArgs& a, hipStream_t s) {
    if (a.kv_map)
        hipLaunchKernelGGL((attn_fwd_f32_kernel<D, true>), grid_for(a, BM), dim3(kThreads), 0, s, a,
                           a.score_scale * kLog2e);
    else
        hipLaunchKernelGGL((attn_fwd_f32_kernel<D, false>), grid_for(a, BM), dim3(kThreads), 0, s, a,
                           a.score_scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

// 256-row eight-wave workgroups when they still give every CU work (counting
// split-K copies); otherwise 128-row four-wave workgroups for parallelism.
bool prefill_uses_eight_waves(const RunArgs& a) {
    const long long wgs256 = static_cast<long long>((a.seq_len + 255) / 256) * a.batch * a.n_heads;
    return wgs256 * (a.n_split > 1 ? a.n_split : 1) >= 256;
}

#define PA_DISPATCH_D(fn, d, ...)                       \
    switch (d) {                                        \
        case 64: return fn<64>(__VA_ARGS__);            \
        case 96: return fn<96>(__VA_ARGS__);            \
        case 128: return fn<128>(__VA_ARGS__);          \
        default: return hipErrorInvalidValue;           \
    }

hipError_t launch_attn_bf16(int head_dim, const RunArgs& a, hipStream_t s) { PA_DISPATCH_D(launch_bf16_d, head_dim, a, s) }
hipError_t launch_attn_i16(int head_dim, const RunArgs& a, hipStream_t s) { PA_DISPATCH_D(launch_i16_d, head_dim, a, s) }
hipError_t launch_attn_i16q(int head_dim, const RunArgs& a, hipStream_t s) { PA_DISPATCH_D(launch_i16q_d, head_dim, a, s) }
hipError_t launch_attn_i16pwl(int head_dim, const RunArgs& a, hipStream_t s) {
    PA_DISPATCH_D(launch_i16pwl_d, head_dim, a, s)
}
hipError_t launch_attn_f32(int head_dim, const RunArgs& a, hipStream_t s) { PA_DISPATCH_D(launch_f32_d, head_dim, a, s) }

hipError_t launch_kv_cache_update(int head_dim, int el, const RunArgs& a, void* dst_k, void* dst_v, hipStream_t s) {
    const uint32_t row_bytes = static_cast<uint32_t>(a.n_kv_heads) * head_dim * el;
    const size_t blocks = static_cast<size_t>(a.batch) * a.seq_len;  // one workgroup per new token
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffu) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kv_cache_update_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, a,
                       row_bytes, static_cast<char*>(dst_k), static_cast<char*>(dst_v));
    return hipGetLastError();
}

namespace {
// The staging width (threads per workgroup) that prefill_attn_run uses for
// int16 inputs of this shape: 512 for eight-wave head_dim 128 launches.
template <int D>
hipError_t launch_rope_d(const RunArgs& a, int n_heads_x, int16_t* dst, hipStream_t s) {
    RunArgs b = a;
    b.k = a.q;
    b.n_heads = n_heads_x;
    b.n_kv_heads = n_heads_x;
    const long long blocks = static_cast<long long>((a.seq_len + BN - 1) / BN) * a.batch * n_heads_x;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 g(static_cast<unsigned>(blocks));
    if (D == 128 && prefill_uses_eight_waves(b))
        hipLaunchKernelGGL((debug_rope_i16_kernel<D, 512>), g, dim3(512), 0, s, b, dst);
    else
        hipLaunchKernelGGL((debug_rope_i16_kernel<D, 256>), g, dim3(256), 0, s, b, dst);
    return hipGetLastError();
}
template <int D>
hipError_t launch_scores_d(const RunArgs& a, int32_t* dst, hipStream_t s) {
    RunArgs b = a;
    b.dbg_scores = dst;
    return launch_int_d<D, I16QK, true>(b, s);
}
template <int D>
hipError_t launch_scores_q_d(const RunArgs& a, int32_t* dst, hipStream_t s) {
    RunArgs b = a;
    b.dbg_scores = dst;
    return launch_int_d<D, I16QuantQK, true>(b, s);
}
}  // namespace

hipError_t launch_debug_rope_i16(int head_dim, const RunArgs& a, int n_heads_x, int16_t* dst, hipStream_t s) {
    PA_DISPATCH_D(launch_rope_d, head_dim, a, n_heads_x, dst, s)
}
hipError_t launch_debug_scores_i32(int head_dim, const RunArgs& a, int32_t* dst, hipStream_t s) {
    PA_DISPATCH_D(launch_scores_d, head_dim, a, dst, s)
}
hipError_t launch_debug_scores_q16(int head_dim, const RunArgs& a, int32_t* dst, hipStream_t s) {
    PA_DISPATCH_D(launch_scores_q_d, head_dim, a, dst, s)
}

}  // namespace pa
