// bf16 fused RoPE causal prefill with K, V and the RoPE table rows of K moved
// from HBM into LDS by the gfx950 direct buffer->LDS loads (no registers, no
// VALU on the way in), for head_dim 64 and 96.
//
// What is computed is the fused prefill attention of "手写内核实现6倍prefill加速"
// §2.2/§3.1 (RoPE of Q and K from position-indexed cos/sin tables inside the
// attention kernel, the rotated K going straight into the dot product), blocked
// with a running max and sum as in the MNN-on-K3 blog §六 and the XNet-DNN
// article §三.3 (FlashAttention-2: Q rows split over waves that share each
// staged K/V tile, rescale deferred to the end).
//
// gfx950 design:
//  * one workgroup = 8 waves x 32 query rows of one (batch, head); 64-key
//    tiles; four LDS stages each for K, V and the table rows of K;
//  * the two wave groups (waves 0-3 and 4-7: one wave of each per SIMD) run
//    half a tile apart: while one issues the matrix work of a tile (P.V of it,
//    Q.K^T of the next) the other runs the vector work (softmax, half of the
//    staging), then they swap at a workgroup barrier -- the matrix core and
//    the vector ALU of a SIMD are fed by different waves;
//  * staging in place in LDS: K(t) -> K' = RoPE(K) in fp16 (the table's fp16
//    (cos, sin) pairs), V(t) bf16 -> fp16, each half tile by one group;
//  * S^T = K'.Q'^T on v_mfma_f32_32x32x16_f16 with Q' (pre-scaled by
//    score_scale * log2 e) held in registers; the MFMA's C operand carries -m,
//    so the scores arrive shifted by the row's running max m;
//  * m is the exact maximum of the first tile; later it moves only when a row
//    sum leaves range, by a whole number of log2 units with O and l scaled by
//    a power of two;
//  * O^T += V^T.P~^T on the fp16 MFMA, V^T read by ds_read_b64_tr_b16 (the
//    transpose happens in the LDS read);
//  * the loop loads nothing into registers, so every wait on the fetches is
//    an explicit s_waitcnt with the exact number of fetch ops allowed to stay
//    in flight.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "device_common.h"
#include "internal.h"

namespace pa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

#define LDS_AS(p) ((__attribute__((address_space(3))) void*)(p))
#define LDS_S4(p) ((__attribute__((address_space(3))) s16x4*)(p))

// Direct buffer -> LDS load, 16 bytes per lane: lane l lands at lds + 16 l
// (M0 = lds).  The host pass of the compiler has no such builtin.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_AS(lds), 16, voff, soff, 0, 0);
#endif
}

constexpr int kThreads8 = 512;
constexpr float kSumLimit = 1073741824.0f;  // 2^30: a row sum past it (or inf) redoes the tile with a raised shift
constexpr int kRsrcWord3 = 0x00020000;      // buffer descriptor word 3 (gfx9: 32-bit data format)

// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (3 << 14)); }

// Workgroup barrier with no memory fence: each wave has already waited for
// its own LDS writes and fetches; the asm keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void wg_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// LDS layout of a 64-key tile of K, V and the table rows of K.  A fetch op
// moves 64 lanes x 16 bytes into 1 KB; src_* give the (row, byte) of the
// source that a destination byte p of the tile holds.  The Q.K^T reads (16
// rows x 16 bytes per pass), transposed V reads (4 rows x 64 bytes) and
// staging accesses (4 rows x 64 bytes) each fall into distinct banks.
//
// head_dim 96: rows packed at 192 bytes (row r at 192 r, which repeats its
// bank offset every 4 rows); the 16-byte chunks of a K row r are XOR-permuted
// by (r >> 2) & 3 inside aligned groups of four, which spreads 16 consecutive
// rows of a Q.K^T read over all banks.
struct L96 {
    static constexpr int kRowB = 192, kTile = 64 * kRowB, kOps = kTile / 1024;
    static constexpr int kKOp = 1024, kVOp = 1024, kTOp = 1024;
    static constexpr int kKBytes = kTile, kVBytes = kTile, kTBytes = kTile;
    __device__ static int kf(int r) { return (r >> 2) & 3; }
    __device__ static void src_k(int p, int& r, int& b) {
        r = p / kRowB;
        b = (((p % kRowB) >> 4) ^ kf(r)) << 4;
    }
    __device__ static void src_v(int p, int& r, int& b) {
        r = p / kRowB;
        b = p % kRowB;
    }
    __device__ static void src_t(int p, int& r, int& b) { src_v(p, r, b); }
    // Q.K^T A operand of row lq, k-step ks, key block blk:
    // qk_base(lq, lh, ks & 1) + 64 (ks >> 1) + kKb blk (the permutation of rows
    // lq and lq + 32 is the same).
    static constexpr int kKb = 32 * kRowB;
    __device__ static int qk_base(int lq, int lh, int e) { return lq * kRowB + 16 * ((2 * e + lh) ^ kf(lq)); }
    // transposed V reads: pv_base + kPvKk kk + kPvHalf half + 64 db
    static constexpr int kPvKk = 16 * kRowB, kPvHalf = 8 * kRowB;
    __device__ static int pv_base(int lane) {
        const int g = lane >> 4, s = lane & 15, lh = lane >> 5;
        return (4 * lh + (s >> 2)) * kRowB + 2 * (16 * (g & 1) + 4 * (s & 3));
    }
    // staging: 8 threads per row of a half tile, piece i at + 64 i, rows 32..63 at + kHalf*
    __device__ static int st_k(int tg) {
        const int r = tg >> 3;
        return r * kRowB + 16 * (((tg & 7) >> 1) ^ kf(r)) + 8 * (tg & 1);
    }
    __device__ static int st_v(int tg) { return (tg >> 3) * kRowB + 8 * (tg & 7); }
    __device__ static int st_t(int tg) { return st_v(tg); }
    static constexpr int kHalfK = 32 * kRowB, kHalfV = 32 * kRowB, kHalfT = 32 * kRowB;
};

// head_dim 64: op j of K and V holds rows j, j + 8, ..., j + 56 (rows r and
// r + 1 in different ops), each op followed by a pad (16 bytes for K, 64 for
// V); the table rows are packed.
struct L64 {
    static constexpr int kRowB = 128, kTile = 64 * kRowB, kOps = kTile / 1024;
    static constexpr int kKOp = 1024 + 16, kVOp = 1024 + 64, kTOp = 1024;
    static constexpr int kKBytes = kOps * kKOp, kVBytes = kOps * kVOp, kTBytes = kTile;
    __device__ static int at(int r, int b, int op) { return (r % kOps) * op + (r / kOps) * kRowB + b; }
    __device__ static void src_k(int p, int& r, int& b) {
        const int j = p >> 10, q = p & 1023;
        r = j + kOps * (q / kRowB);
        b = q % kRowB;
    }
    __device__ static void src_v(int p, int& r, int& b) { src_k(p, r, b); }
    __device__ static void src_t(int p, int& r, int& b) {
        r = p / kRowB;
        b = p % kRowB;
    }
    static constexpr int kKb = (32 / kOps) * kRowB;
    __device__ static int qk_base(int lq, int lh, int e) { return at(lq, 16 * lh + 32 * e, kKOp); }
    static constexpr int kPvKk = (16 / kOps) * kRowB, kPvHalf = kRowB;
    __device__ static int pv_base(int lane) {
        const int g = lane >> 4, s = lane & 15, lh = lane >> 5;
        return at(4 * lh + (s >> 2), 2 * (16 * (g & 1) + 4 * (s & 3)), kVOp);
    }
    __device__ static int st_k(int tg) { return at(tg >> 3, 8 * (tg & 7), kKOp); }
    __device__ static int st_v(int tg) { return at(tg >> 3, 8 * (tg & 7), kVOp); }
    __device__ static int st_t(int tg) { return (tg >> 3) * kRowB + 8 * (tg & 7); }
    static constexpr int kHalfK = (32 / kOps) * kRowB, kHalfV = (32 / kOps) * kRowB, kHalfT = 32 * kRowB;
};

template <int D>
struct LayoutOf;
template <>
struct LayoutOf<64> {
    using type = L64;
};
template <>
struct LayoutOf<96> {
    using type = L96;
};

// The two wave groups of a workgroup (waves 0-3 = A, waves 4-7 = B; waves w
// and w + 4 share a SIMD) run half a tile apart.  A tile's work for one wave
// splits into a vector phase -- softmax of S(t) (exp2, fp16 P~, row sums),
// half of the staging -- and a matrix phase -- O^T += V^T(t).P~(t)^T and
// S(t+1) = K'(t+1).Q'^T.  Half-step h ends with a workgroup barrier; group A
// runs the vector phase of tile h/2 at even h and its matrix phase at odd h,
// group B the reverse.  Tile x by half-step:
//   h = 2x-7   K(x), table(x) fetched (A)      h = 2x-5   V(x) fetched (B)
//   h = 2x-3   K(x) rows 0-31 rotated (B)      h = 2x-2   rows 32-63 (A)
//   h = 2x-1   V(x) rows 0-31 converted (B)    h = 2x     rows 32-63 (A)
//   h = 2x-1, 2x      K'(x) read by Q.K^T (A, then B)
//   h = 2x+1, 2x+2    V(x) read by P.V (A, then B)
// so four LDS stages per tensor hold every tile from its fetch to its last
// read.  A fetch is waited for at the end of the even half-step before its
// first use, by the group that issued it: A with the 2 NQ ops of its latest
// fetch still in flight, B with the NQ ops of its latest.
template <int D>
struct PingPong {
    using L = typename LayoutOf<D>::type;
    static constexpr int NS = 4;            // LDS stages per tensor
    static constexpr int KS = D / 16;       // 16-deep k-steps of Q.K^T
    static constexpr int DB = D / 32;       // 32-dim blocks of O
    static constexpr int RP = D / 32;       // 8-byte pieces per thread in a half-tile staging pass
    static constexpr int NQ = L::kOps / 4;  // fetch ops per wave per tensor tile (4 waves fetch a tile)

    char* kbuf[NS];
    char* vbuf[NS];
    char* tbuf[NS];

    int S, q0, qw0, w, wg, lane, lq, lh;
    int n_all;   // key tiles the workgroup stages
    int n_full;  // tiles every row of the workgroup sees whole
    int n_dma;   // tiles that lie inside the sequence
    __amdgpu_buffer_rsrc_t rk, rv, rt;  // K, V of this (batch, kv head) from token 0; the table from position off
    uint32_t gstride;                   // bytes between consecutive tokens of K / V
    uint32_t k_vo[NQ], v_vo[NQ], t_vo[NQ];  // this lane's source offsets in its fetch ops of tile 0
    int qk_b[2], pv_off, st_k, st_v, st_t;

    f16x8 q[KS];
    f32x16 o[DB];
    f32x16 bias;
    f32x16 s[2];
    uint32_t pk[16];
    float l_a, l_b;

    // ------------------------------------------------------------ fetches

    // This wave's share of the fetch of K(t) and its table rows into stage
    // ST.  CLAMP: the tile reaches past the sequence; its rows are clamped to
    // the last token (those keys are masked for every query).
    template <int ST, bool CLAMP>
    __device__ __forceinline__ void fetch_kt(int t) const {
        if (!CLAMP) {
            const uint32_t sk = static_cast<uint32_t>(t) * BN * gstride;
            const uint32_t st = static_cast<uint32_t>(t) * BN * L::kRowB;
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int j = wg * NQ + i;
                dma16(rk, kbuf[ST] + j * L::kKOp, k_vo[i], sk);
                dma16(rt, tbuf[ST] + j * L::kTOp, t_vo[i], st);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int j = wg * NQ + i, p = j * 1024 + 16 * lane;
                int r, b;
                L::src_k(p, r, b);
                r = min(t * BN + r, S - 1);
                dma16(rk, kbuf[ST] + j * L::kKOp, static_cast<uint32_t>(r) * gstride + b, 0);
                L::src_t(p, r, b);
                r = min(t * BN + r, S - 1);
                dma16(rt, tbuf[ST] + j * L::kTOp, static_cast<uint32_t>(r) * L::kRowB + b, 0);
            }
        }
    }
    template <int ST, bool CLAMP>
    __device__ __forceinline__ void fetch_v(int t) const {
        if (!CLAMP) {
            const uint32_t sv = static_cast<uint32_t>(t) * BN * gstride;
#pragma unroll
            for (int i = 0; i < NQ; ++i) dma16(rv, vbuf[ST] + (wg * NQ + i) * L::kVOp, v_vo[i], sv);
        } else {
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int j = wg * NQ + i;
                int r, b;
                L::src_v(j * 1024 + 16 * lane, r, b);
                r = min(t * BN + r, S - 1);
                dma16(rv, vbuf[ST] + j * L::kVOp, static_cast<uint32_t>(r) * gstride + b, 0);
            }
        }
    }
    // Fetch of K(t) / V(t) if the tile exists; returns whether ops were issued.
    template <int ST, bool STEADY>
    __device__ __forceinline__ bool fetch_kt_if(int t) const {
        if (STEADY || t < n_dma) {
            fetch_kt<ST, false>(t);
            return true;
        }
        if (t < n_all) {
            fetch_kt<ST, true>(t);
            return true;
        }
        return false;
    }
    template <int ST, bool STEADY>
    __device__ __forceinline__ bool fetch_v_if(int t) const {
        if (STEADY || t < n_dma) {
            fetch_v<ST, false>(t);
            return true;
        }
        if (t < n_all) {
            fetch_v<ST, true>(t);
            return true;
        }
        return false;
    }

    // ------------------------------------------------------------ staging

    // A half tile (rows 32Y..32Y+31) staged in place: this thread's raw K, V
    // and table pieces are read first (their LDS latency hides behind the
    // softmax), then K' = RoPE(K) and V -> fp16 are written back.
    struct Stage {
        uint2 k[RP], v[RP], t[RP];
    };
    template <int SK, int SV, int Y, bool DO_K, bool DO_V>
    __device__ __forceinline__ void stage_read(Stage& r) const {
        const char* kp = kbuf[SK] + st_k + Y * L::kHalfK;
        const char* tp = tbuf[SK] + st_t + Y * L::kHalfT;
        const char* vp = vbuf[SV] + st_v + Y * L::kHalfV;
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            if (DO_K) {
                r.k[i] = *reinterpret_cast<const uint2*>(kp + 64 * i);
                r.t[i] = *reinterpret_cast<const uint2*>(tp + 64 * i);
            }
            if (DO_V) r.v[i] = *reinterpret_cast<const uint2*>(vp + 64 * i);
        }
    }
    template <int SK, int SV, int Y, bool DO_K, bool DO_V>
    __device__ __forceinline__ void stage_write(const Stage& r) const {
        char* kp = kbuf[SK] + st_k + Y * L::kHalfK;
        char* vp = vbuf[SV] + st_v + Y * L::kHalfV;
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            if (DO_K)
                *reinterpret_cast<uint2*>(kp + 64 * i) =
                    make_uint2(rot_pack_h2h(bf_lo(r.k[i].x), bf_hi(r.k[i].x), r.t[i].x),
                               rot_pack_h2h(bf_lo(r.k[i].y), bf_hi(r.k[i].y), r.t[i].y));
            if (DO_V)
                *reinterpret_cast<uint2*>(vp + 64 * i) =
                    make_uint2(pack_h2(bf_lo(r.v[i].x), bf_hi(r.v[i].x)), pack_h2(bf_lo(r.v[i].y), bf_hi(r.v[i].y)));
        }
    }
    template <int SK, int SV, int Y, bool DO_K, bool DO_V>
    __device__ __forceinline__ void stage_now() const {
        Stage r;
        stage_read<SK, SV, Y, DO_K, DO_V>(r);
        stage_write<SK, SV, Y, DO_K, DO_V>(r);
    }

    // ------------------------------------------------------------ matrix products

    // Active 32-key blocks of tile t for this wave (0, 1 or 2; wave-uniform).
    __device__ __forceinline__ int nact(int t) const {
        const int last = min(qw0 + 31, S - 1);
        if (qw0 >= S || t < 0) return 0;
        const int kt0 = t * BN;
        return kt0 + 32 <= last ? 2 : (kt0 <= last ? 1 : 0);
    }

    __device__ __forceinline__ f16x8 kfrag(const char* kb, int blk, int ks) const {
        return *reinterpret_cast<const f16x8*>(kb + qk_b[ks & 1] + 64 * (ks >> 1) + blk * L::kKb);
    }
    // S^T = K'.Q'^T of the tile in stage ST (nb blocks of 32 keys), shifted by
    // the C operand; the two blocks' dependent MFMA chains are interleaved.
    template <int ST>
    __device__ __forceinline__ void qk(int nb, const f32x16& c) {
        const char* kb = kbuf[ST];
        if (nb == 2) {
            f16x8 a0[KS], a1[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                a0[ks] = kfrag(kb, 0, ks);
                a1[ks] = kfrag(kb, 1, ks);
            }
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[0], q[0], c, 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[0], q[0], c, 0, 0, 0);
#pragma unroll
            for (int ks = 1; ks < KS; ++ks) {
                s[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[ks], q[ks], s[0], 0, 0, 0);
                s[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[ks], q[ks], s[1], 0, 0, 0);
            }
        } else if (nb == 1) {
            f16x8 a0[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) a0[ks] = kfrag(kb, 0, ks);
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[0], q[0], c, 0, 0, 0);
#pragma unroll
            for (int ks = 1; ks < KS; ++ks) s[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[ks], q[ks], s[0], 0, 0, 0);
        }
    }

    // V^T operands of the 16-key step kk of the tile in stage ST: for each
    // 32-dim block, keys 16kk + 4lh + (0..3) and 16kk + 8 + 4lh + (0..3) of dim
    // 32db + (lane % 32), transposed by the LDS read.
    template <int ST>
    __device__ __forceinline__ void read_v(int kk, f16x8* a) const {
        const char* base = vbuf[ST] + pv_off + kk * L::kPvKk;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_S4(base + 64 * db));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_S4(base + 64 * db + L::kPvHalf));
            const s16x4 both[2] = {lo, hi};
            a[db] = __builtin_bit_cast(f16x8, both);
        }
    }
    // O^T += V^T . P~^T for the 16-key step kk.
    __device__ __forceinline__ void mfma_v(int kk, const f16x8* a) {
        const u32x4 b4 = {pk[4 * kk], pk[4 * kk + 1], pk[4 * kk + 2], pk[4 * kk + 3]};
        const f16x8 p = __builtin_bit_cast(f16x8, b4);
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[db], p, o[db], 0, 0, 0);
    }
    // P.V of the na active key blocks of the tile in stage ST, operand reads one k-step ahead.
    template <int ST>
    __device__ __forceinline__ void pv(int na) {
        f16x8 va[DB], vb[DB];
        read_v<ST>(0, va);
        if (na == 2) {
            read_v<ST>(1, vb);
            mfma_v(0, va);
            read_v<ST>(2, va);
            mfma_v(1, vb);
            read_v<ST>(3, vb);
            mfma_v(2, va);
            mfma_v(3, vb);
        } else if (na == 1) {
            read_v<ST>(1, vb);
            mfma_v(0, va);
            mfma_v(1, vb);
        }
    }

    // ------------------------------------------------------------ softmax

    // Causal mask of the diagonal block: key acc_row(v, lh) > query lq.
    __device__ __forceinline__ void mask_diag(f32x16& x) const {
#pragma unroll
        for (int v = 0; v < 16; ++v)
            if (acc_row(v, lh) > lq) x[v] = kNegInf;
    }

    // P~ = exp2(S) of the na active key blocks as fp16 pairs, added into the
    // row sums.  All exponentials issue first (the transcendental unit's
    // latency then hides behind its own queue), the packs and sums after.
    __device__ __forceinline__ void exp_tile(int na) {
        const f16x2 ones = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
        f32x16 e[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            if (kb < na) {
#pragma unroll
                for (int v = 0; v < 16; ++v) e[kb][v] = fast_exp2(s[kb][v]);
            }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            if (kb < na) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t h = pack_h2(e[kb][2 * j], e[kb][2 * j + 1]);
                    pk[8 * kb + j] = h;
                    if (j & 1)
                        l_b = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, h), ones, l_b, false);
                    else
                        l_a = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, h), ones, l_a, false);
                }
            }
    }

    __device__ __forceinline__ float tile_max(int na) const {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            if (kb < na) {
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
            }
        return halves_max(mx);
    }

    // Softmax of tile t (na active blocks) into pk.  FIRST: the shift becomes
    // the tile's exact row maximum.  Otherwise the shift stays put; if a row's
    // sum leaves kSumLimit (an fp16 P~ overflowed, or the sum grew too large)
    // the tile is redone with the shift moved up by a whole number d of log2
    // units -- enough to bring the tile's maximum to 0 or below and the
    // previous sum under 2^20 -- and O, l and the C operand scaled by 2^-d: a
    // power of two, so the rescale rounds nothing, and any shift at or below
    // the true maximum gives the same normalised result.
    template <bool FULL, bool FIRST>
    __device__ __forceinline__ void softmax(int t, int na) {
        if (!FULL) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                if (kb < na && t * BN + 32 * kb == qw0) mask_diag(s[kb]);
        }
        if (FIRST) {
            const float mx = tile_max(na);
#pragma unroll
            for (int v = 0; v < 16; ++v) bias[v] = -mx;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                if (kb < na) s[kb] -= mx;
        }
        const float la0 = l_a, lb0 = l_b;
        exp_tile(na);
        if (FULL) {
            __builtin_amdgcn_sched_group_barrier(0x400, 32, 0);  // exponentials
            __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);  // packs, sums
        }
        if (!FIRST && __builtin_amdgcn_ballot_w64(!(fmaxf(l_a, l_b) < kSumLimit)) != 0) {
            const float mx = tile_max(na);
            const float lm = halves_max(fmaxf(la0, lb0));  // < 2 kSumLimit: the previous tile passed the test
            const int e_l = static_cast<int>((__float_as_uint(lm) >> 23) & 255) - 127 - 20;
            const int dv = max(max(mx > 0.f ? static_cast<int>(__builtin_ceilf(mx)) : 0, e_l), 0);
            const float d = static_cast<float>(dv);
            const float alpha = __builtin_amdgcn_ldexpf(1.0f, -dv);
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] *= alpha;
            l_a = la0 * alpha;
            l_b = lb0 * alpha;
#pragma unroll
            for (int v = 0; v < 16; ++v) bias[v] -= d;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                if (kb < na) s[kb] -= d;
            exp_tile(na);
        }
    }

    // ------------------------------------------------------------ half-steps

    // Vector phase of tile t for group A (even half-step 2t): softmax of tile
    // t, RoPE of K(t+1) rows 32-63, V(t) rows 32-63 -> fp16.  Ends having
    // waited for its fetch of K(t+2) and table(t+2) (group B rotates rows 0-31
    // of K(t+2) next); the fetch of tile t+3, if any, stays in flight.
    template <int TS, bool STEADY, bool FIRST = false>
    __device__ __forceinline__ void valu_a(int t) {
        constexpr int S1 = (TS + 1) % NS;
        const int na = STEADY ? 2 : nact(t);
        const bool dk = STEADY || t + 1 < n_all;
        Stage r;
        if (dk)
            stage_read<S1, TS, 1, true, true>(r);
        else
            stage_read<S1, TS, 1, false, true>(r);
        __builtin_amdgcn_sched_barrier(0);
        if (STEADY || na > 0) softmax<STEADY, FIRST>(t, na);
        if (dk)
            stage_write<S1, TS, 1, true, true>(r);
        else
            stage_write<S1, TS, 1, false, true>(r);
        if (STEADY || t + 3 < n_all)
            wait_vm_lgkm0<2 * NQ>();
        else
            wait_vm_lgkm0<0>();
        wg_barrier();
    }
    // Matrix phase of tile t for group A (odd half-step 2t+1): fetch of K(t+4)
    // and table(t+4), P.V(t), Q.K^T(t+1).
    template <int TS, bool STEADY>
    __device__ __forceinline__ void mfma_a(int t) {
        constexpr int S1 = (TS + 1) % NS;
        __builtin_amdgcn_s_setprio(1);  // the matrix-phase wave issues first on its SIMD
        fetch_kt_if<TS, STEADY>(t + 4);
        const int na = STEADY ? 2 : nact(t);
        const int na1 = STEADY ? 2 : (t + 1 < n_all ? nact(t + 1) : 0);
        if (STEADY || na > 0) pv<TS>(na);
        if (STEADY || na1 > 0) qk<S1>(na1, bias);
        if (STEADY) mfma_order(true);
        __builtin_amdgcn_s_setprio(0);
        wait_lgkm0();
        wg_barrier();
    }
    // Matrix phase of tile t-1 for group B (even half-step 2t): P.V(t-1),
    // Q.K^T(t).  Ends having waited for its fetch of V(t+1); the fetch of
    // V(t+2), if any, stays in flight.
    template <int TS, bool STEADY>
    __device__ __forceinline__ void mfma_b(int t) {
        constexpr int SP = (TS + NS - 1) % NS;
        __builtin_amdgcn_s_setprio(1);
        const int nap = STEADY ? 2 : nact(t - 1);
        const int na = STEADY ? 2 : nact(t);
        if (STEADY || nap > 0) pv<SP>(nap);
        if (STEADY || na > 0) qk<TS>(na, bias);
        if (STEADY) mfma_order(false);
        __builtin_amdgcn_s_setprio(0);
        if (STEADY || t + 2 < n_all)
            wait_vm_lgkm0<NQ>();
        else
            wait_vm_lgkm0<0>();
        wg_barrier();
    }
    // Vector phase of tile t for group B (odd half-step 2t+1): fetch of V(t+3),
    // softmax of tile t, RoPE of K(t+2) rows 0-31, V(t+1) rows 0-31 -> fp16.
    template <int TS, bool STEADY, bool FIRST = false>
    __device__ __forceinline__ void valu_b(int t) {
        constexpr int S1 = (TS + 1) % NS, S2 = (TS + 2) % NS, S3 = (TS + 3) % NS;
        fetch_v_if<S3, STEADY>(t + 3);
        const int na = STEADY ? 2 : nact(t);
        const bool dk = STEADY || t + 2 < n_all, dv = STEADY || t + 1 < n_all;
        Stage r;
        if (dk)
            stage_read<S2, S1, 0, true, true>(r);
        else if (dv)
            stage_read<S2, S1, 0, false, true>(r);
        __builtin_amdgcn_sched_barrier(0);
        if (STEADY || na > 0) softmax<STEADY, FIRST>(t, na);
        if (dk)
            stage_write<S2, S1, 0, true, true>(r);
        else if (dv)
            stage_write<S2, S1, 0, false, true>(r);
        wait_lgkm0();
        wg_barrier();
    }

    // Issue order of a full matrix phase (P.V of two blocks, Q.K^T of two
    // blocks): operand reads stream ahead of their MFMAs so only a few
    // fragments are live at a time; group A's fetch ops go out between MFMAs.
    __device__ __forceinline__ static void mfma_order(bool fetch) {
        if (fetch) __builtin_amdgcn_sched_group_barrier(0x020, NQ, 0);  // buffer loads -> LDS
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * DB, 0);          // V^T reads, k-step 0
#pragma unroll
        for (int kk = 0; kk < 3; ++kk) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * DB, 0);  // next k-step's reads
#pragma unroll
            for (int db = 0; db < DB; ++db) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // K' fragments ks 0, 1 of both blocks
        if (fetch) __builtin_amdgcn_sched_group_barrier(0x020, NQ, 0);
#pragma unroll
        for (int db = 0; db < DB; ++db) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 2 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
    }

    // Group A: vector phase at even half-steps, matrix phase at odd ones.
    // Steady groups of four tiles need every tile they touch whole for all
    // rows and every tile they fetch inside the sequence.
    __device__ __forceinline__ void loop_a() {
        valu_a<0, false, true>(0);
        mfma_a<0, false>(0);
        int t = 1;
        for (; t + 4 < n_full && t + 7 < n_dma; t += 4) {
            valu_a<1, true>(t);
            mfma_a<1, true>(t);
            valu_a<2, true>(t + 1);
            mfma_a<2, true>(t + 1);
            valu_a<3, true>(t + 2);
            mfma_a<3, true>(t + 2);
            valu_a<0, true>(t + 3);
            mfma_a<0, true>(t + 3);
        }
        for (; t < n_all; t += 4) {
            valu_a<1, false>(t);
            mfma_a<1, false>(t);
            if (t + 1 < n_all) {
                valu_a<2, false>(t + 1);
                mfma_a<2, false>(t + 1);
            }
            if (t + 2 < n_all) {
                valu_a<3, false>(t + 2);
                mfma_a<3, false>(t + 2);
            }
            if (t + 3 < n_all) {
                valu_a<0, false>(t + 3);
                mfma_a<0, false>(t + 3);
            }
        }
    }
    // Group B: matrix phase at even half-steps (for the tile before), vector
    // phase at odd ones; its last P.V (half-step 2 n_all) needs no barrier.
    __device__ __forceinline__ void loop_b() {
        mfma_b<0, false>(0);
        valu_b<0, false, true>(0);
        int t = 1;
        for (; t + 4 < n_full && t + 7 < n_dma; t += 4) {
            mfma_b<1, true>(t);
            valu_b<1, true>(t);
            mfma_b<2, true>(t + 1);
            valu_b<2, true>(t + 1);
            mfma_b<3, true>(t + 2);
            valu_b<3, true>(t + 2);
            mfma_b<0, true>(t + 3);
            valu_b<0, true>(t + 3);
        }
        for (; t < n_all; t += 4) {
            mfma_b<1, false>(t);
            valu_b<1, false>(t);
            if (t + 1 < n_all) {
                mfma_b<2, false>(t + 1);
                valu_b<2, false>(t + 1);
            }
            if (t + 2 < n_all) {
                mfma_b<3, false>(t + 2);
                valu_b<3, false>(t + 2);
            }
            if (t + 3 < n_all) {
                mfma_b<0, false>(t + 3);
                valu_b<0, false>(t + 3);
            }
        }
        const int tl = n_all - 1;
        const int nl = nact(tl);
        if (nl > 0) {
            switch (tl & 3) {
                case 0: pv<0>(nl); break;
                case 1: pv<1>(nl); break;
                case 2: pv<2>(nl); break;
                default: pv<3>(nl); break;
            }
        }
    }

    __device__ __forceinline__ void load_q(const RunArgs& a, int b, int hq, int off, float scale) {
        const int qi = qw0 + lq;
        const bool ok = qi < S;
        const char* qrow = static_cast<const char*>(a.q) +
                           ((static_cast<size_t>(b) * S + (ok ? qi : 0)) * a.n_heads + hq) * D * 2;
        const char* tab = reinterpret_cast<const char*>(a.rope_h2 + (static_cast<size_t>(off) + (ok ? qi : 0)) * (D / 2));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = 16 * ks + 8 * lh;
            uint4 raw = make_uint4(0, 0, 0, 0), cs = raw;
            if (ok) {
                raw = *reinterpret_cast<const uint4*>(qrow + 2 * d0);
                cs = *reinterpret_cast<const uint4*>(tab + 2 * d0);
            }
            const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
            const uint32_t tv[4] = {cs.x, cs.y, cs.z, cs.w};
            uint32_t r[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float x = bf_lo(wv[j]), y = bf_hi(wv[j]);
                const float c = h_lo(tv[j]), sn = h_hi(tv[j]);
                r[j] = pack_h2(fmaf(x, c, -y * sn) * scale, fmaf(x, sn, y * c) * scale);
            }
            q[ks] = __builtin_bit_cast(f16x8, make_uint4(r[0], r[1], r[2], r[3]));
        }
    }

    // One 256-row query block of (b, hq).
    __device__ __forceinline__ void run(const RunArgs& a, int qb, int b, int hq, float scale) {
        qb = __builtin_amdgcn_readfirstlane(qb);
        b = __builtin_amdgcn_readfirstlane(b);
        hq = __builtin_amdgcn_readfirstlane(hq);
        lane = threadIdx.x & 63;
        w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
        const int grp = w >> 2;
        wg = w & 3;
        lq = lane & 31;
        lh = lane >> 5;
        S = a.seq_len;
        q0 = qb * 256;
        qw0 = q0 + 32 * w;
        const int off = __builtin_amdgcn_readfirstlane(a.pos_offsets ? a.pos_offsets[b] : 0);
        const int hkv = __builtin_amdgcn_readfirstlane(hq / (a.n_heads / a.n_kv_heads));
        n_all = (min(q0 + 256, S) + BN - 1) / BN;
        n_full = q0 / BN;
        n_dma = S / BN;
        gstride = static_cast<uint32_t>(a.n_kv_heads * D * 2);
        const size_t kv0 = (static_cast<size_t>(b) * S * a.n_kv_heads + hkv) * D * 2;
        const uint32_t kv_bytes = static_cast<uint32_t>(S) * gstride;  // < 2^31 (checked at launch)
        rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(static_cast<const char*>(a.k) + kv0), 0, kv_bytes,
                                               kRsrcWord3);
        rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(static_cast<const char*>(a.v) + kv0), 0, kv_bytes,
                                               kRsrcWord3);
        rt = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(a.rope_h2 + static_cast<size_t>(off) * (D / 2)), 0,
                                               static_cast<uint32_t>(S) * L::kRowB, kRsrcWord3);

        // Per-lane constants: fetch sources, LDS read offsets, staging pieces.
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int p = (wg * NQ + i) * 1024 + 16 * lane;
            int r, bb;
            L::src_k(p, r, bb);
            k_vo[i] = static_cast<uint32_t>(r) * gstride + bb;
            L::src_v(p, r, bb);
            v_vo[i] = static_cast<uint32_t>(r) * gstride + bb;
            L::src_t(p, r, bb);
            t_vo[i] = static_cast<uint32_t>(r) * L::kRowB + bb;
        }
        qk_b[0] = L::qk_base(lq, lh, 0);
        qk_b[1] = L::qk_base(lq, lh, 1);
        pv_off = L::pv_base(lane);
        const int tg = threadIdx.x & 255;  // thread within the group
        st_k = L::st_k(tg);
        st_v = L::st_v(tg);
        st_t = L::st_t(tg);

        // Prologue.  Group A fetches K and the table rows of tiles 0..3, group
        // B V(0..2) -- the fetches of half-steps before the loop.  Then K(0)
        // is rotated (rows 0-31 by B, 32-63 by A), and B also rotates rows
        // 0-31 of K(1) and converts rows 0-31 of V(0).
        if (grp == 0) {
            fetch_kt_if<0, false>(0);
            fetch_kt_if<1, false>(1);
            fetch_kt_if<2, false>(2);
            fetch_kt_if<3, false>(3);
        } else {
            fetch_v_if<0, false>(0);
            fetch_v_if<1, false>(1);
            fetch_v_if<2, false>(2);
        }
        load_q(a, b, hq, off, scale);
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = f32x16{};
        l_a = 0.f;
        l_b = 0.f;
        bias = f32x16{};
        wait_vm_lgkm0<0>();
        wg_barrier();
        if (grp == 0) {
            stage_now<0, 0, 1, true, false>();
        } else {
            stage_now<0, 0, 0, true, true>();
            if (1 < n_all) stage_now<1, 0, 0, true, false>();
        }
        wait_lgkm0();
        wg_barrier();
        // S(0) for group A (group B forms it in half-step 0)
        if (grp == 0) {
            const int na0 = nact(0);
            if (na0 > 0) qk<0>(na0, bias);
            loop_a();
        } else {
            loop_b();
        }
        wait_vm_lgkm0<0>();  // no fetch outlives the block: the next block reuses the stages

        // Epilogue: O / l, fp32 rows.
        if (qw0 >= S) return;
        const float inv = 1.0f / halves_sum(l_a + l_b);
        const int qi = qw0 + lq;
        if (qi < S) {
            float* orow = a.out + ((static_cast<size_t>(b) * S + qi) * a.n_heads + hq) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<float4*>(orow + 32 * db + 8 * g + 4 * lh) =
                        make_float4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                                    o[db][4 * g + 3] * inv);
        }
    }
};

template <int D>
__global__ __launch_bounds__(kThreads8, 1) void prefill_bf16_kernel(RunArgs a, float logit_scale) {
    using L = typename LayoutOf<D>::type;
    __shared__ __attribute__((aligned(16))) char k0[L::kKBytes], k1[L::kKBytes], k2[L::kKBytes], k3[L::kKBytes];
    __shared__ __attribute__((aligned(16))) char v0[L::kVBytes], v1[L::kVBytes], v2[L::kVBytes], v3[L::kVBytes];
    __shared__ __attribute__((aligned(16))) char t0[L::kTBytes], t1[L::kTBytes], t2[L::kTBytes], t3[L::kTBytes];
    PingPong<D> p;
    p.kbuf[0] = k0;
    p.kbuf[1] = k1;
    p.kbuf[2] = k2;
    p.kbuf[3] = k3;
    p.vbuf[0] = v0;
    p.vbuf[1] = v1;
    p.vbuf[2] = v2;
    p.vbuf[3] = v3;
    p.tbuf[0] = t0;
    p.tbuf[1] = t1;
    p.tbuf[2] = t2;
    p.tbuf[3] = t3;

    const int n_qblocks = (a.seq_len + 255) / 256;
    const int bid = static_cast<int>(blockIdx.x);
    const bool paired = a.paired != 0;
    for (int item = 0; item < (paired ? 2 : 1); ++item) {
        const BlockPos bp = paired ? map_pair(n_qblocks, a.batch, a.n_heads, bid, item)
                                   : map_block(n_qblocks, a.batch, a.n_heads, bid);
        if (item == 1 && 2 * bp.qb == n_qblocks - 1) break;  // the middle block of an odd count runs once
        const int off = a.pos_offsets ? a.pos_offsets[bp.b] : 0;
        const long long end = static_cast<long long>(off) + a.seq_len;
        if (off < 0 || end > a.max_seq) {
            // positions outside the table: O = 0 for the block, status set
            const int rows = min(256, a.seq_len - bp.qb * 256);
            for (int idx = threadIdx.x; idx < rows * (D / 4); idx += kThreads8) {
                const int r = idx / (D / 4), col = idx % (D / 4);
                float* dst =
                    a.out + ((static_cast<size_t>(bp.b) * a.seq_len + bp.qb * 256 + r) * a.n_heads + bp.hq) * D;
                reinterpret_cast<float4*>(dst)[col] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            if (threadIdx.x == 0) atomicOr(a.status, 1);
            continue;
        }
        if (item == 1) wg_barrier();  // the first block's LDS reads are done
        p.run(a, bp.qb, bp.b, bp.hq, logit_scale);
    }
}

template <int D>
hipError_t launch_d(const RunArgs& a, hipStream_t s) {
    const unsigned n_qb = static_cast<unsigned>((a.seq_len + 255) / 256);
    dim3 g(n_qb * a.batch * a.n_heads);
    RunArgs b = a;
    b.paired = 0;
    if (use_pairs(a)) {
        b.paired = 1;
        g.x = (n_qb + 1) / 2 * a.batch * a.n_heads;
    }
    hipLaunchKernelGGL((prefill_bf16_kernel<D>), g, dim3(kThreads8), 0, s, b, a.score_scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

bool prefill_lds_supported(int head_dim, const RunArgs& a) {
    // buffer offsets are 32-bit: one (batch, kv head) slice of K / V below 2 GiB
    const long long slice = static_cast<long long>(a.seq_len) * a.n_kv_heads * head_dim * 2;
    return (head_dim == 64 || head_dim == 96) && !a.kv_map && a.n_split <= 1 && prefill_uses_eight_waves(a) &&
           slice < (1LL << 31);
}

hipError_t launch_prefill_lds(int head_dim, const RunArgs& a, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_d<64>(a, s);
        case 96: return launch_d<96>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
