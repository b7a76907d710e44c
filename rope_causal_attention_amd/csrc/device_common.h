// Device helpers shared by the prefill kernels (gfx950): operand types,
// bf16 / fp16 conversions, the fp16 RoPE rotation, lane-half reductions and
// the workgroup -> (query block, batch, head) maps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int BN = 64;           // keys per LDS tile
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -__builtin_huge_valf();

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ int i16_lo(uint32_t w) { return static_cast<int>(w << 16) >> 16; }
__device__ __forceinline__ int i16_hi(uint32_t w) { return static_cast<int>(w) >> 16; }

// Two fp32 -> packed fp16, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    f16x2 h = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    return __builtin_bit_cast(uint32_t, h);
}

// Rotated pair (x c - y s, x s + y c) packed as two fp16, with the table's
// fp16 (cos, sin) pair in one word (cos in the low half).  v_fma_mix takes the
// fp16 halves as sources directly: the products y s and y c are formed and
// rounded in fp32, and each fused multiply-add then rounds once, straight to
// fp16.  Spelled out so that every copy of the staging code rounds K' the
// same way: left to itself the compiler fuses the fp16 conversion into the
// FMA in some copies and not in others, which would make K' depend on which
// pipeline step staged the tile.
__device__ __forceinline__ uint32_t rot_pack_h2h(float x, float y, uint32_t cs) {
    float ys, yc;
    asm("v_fma_mix_f32 %0, -%1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(ys) : "v"(y), "v"(cs));
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(yc) : "v"(y), "v"(cs));
    uint32_t r;
    asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(x), "v"(cs), "v"(ys));
    asm("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(r) : "v"(x), "v"(cs), "v"(yc));
    return r;
}
// Range guards of the narrowing conversions; bad() is this thread's verdict.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
// fp16 results (packed pairs): the running maximum of their magnitude bits;
// a half at 0x7c00 or above is inf or NaN (the value left the fp16 range).
struct F16Guard {
    uint32_t m = 0;
    __device__ __forceinline__ void add(uint32_t h2) {
        m = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, m),
                                                                   __builtin_bit_cast(u16x2, h2 & 0x7fff7fffu)));
    }
    __device__ __forceinline__ bool bad() const { return (m & 0xffffu) >= 0x7c00u || (m >> 16) >= 0x7c00u; }
};
// Rotated int16 values split into int8 digits h and l (a = 128 h + l,
// l in [-64, 63]): both fit int8 for every a in [-16448, 16319].
constexpr int kDigitMax = 16319, kDigitMin = -16448;
struct DigitGuard {
    int mx = 0, mn = 0;
    __device__ __forceinline__ void add(int a, int b) {
        mx = max(mx, max(a, b));
        mn = min(mn, min(a, b));
    }
    __device__ __forceinline__ bool bad() const { return mx > kDigitMax || mn < kDigitMin; }
};
// Inputs that cannot leave the range (codes quantised to [-2048, 2047]).
struct NoGuard {
    __device__ __forceinline__ void add(int, int) {}
    __device__ __forceinline__ bool bad() const { return false; }
};

// The same rotation from fp32 (cos, sin): (x c - y s, x s + y c), the product
// y s (and y c) rounded to fp32 and one fused multiply-add rounding once to
// fp16, as rot_pack_h2h.
__device__ __forceinline__ uint32_t rot_pack_f32(float x, float y, float c, float s) {
    const float ys = -y * s, yc = y * c;
    uint32_t r;
    asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[0,0,0]" : "=v"(r) : "v"(x), "v"(c), "v"(ys));
    asm("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel_hi:[0,0,0]" : "+v"(r) : "v"(x), "v"(s), "v"(yc));
    return r;
}

__device__ __forceinline__ float h_lo(uint32_t w) { return static_cast<float>(__builtin_bit_cast(f16x2, w)[0]); }
__device__ __forceinline__ float h_hi(uint32_t w) { return static_cast<float>(__builtin_bit_cast(f16x2, w)[1]); }

// Combine a per-lane value with the same lane of the other 32-lane half.
__device__ __forceinline__ float halves_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row index of accumulator element v (0..15) of a 32x32 MFMA result for lane
// half lh: rows come in groups of 4, interleaved between the two halves.
__device__ __forceinline__ int acc_row(int v, int lh) { return 8 * (v >> 2) + 4 * lh + (v & 3); }

// 16-byte load at a byte offset from a workgroup-uniform base (32-bit offset).
__device__ __forceinline__ uint4 ld16(const char* base, uint32_t off) {
    return *reinterpret_cast<const uint4*>(base + off);
}
__device__ __forceinline__ float4 ld16f(const char* base, uint32_t off) {
    return *reinterpret_cast<const float4*>(base + off);
}

// Work order: longest query blocks first; when the (batch, head) count is a
// multiple of 8, consecutive workgroup ids (dealt round-robin to the 8 XCDs)
// are mapped so that each XCD owns a contiguous range of (batch, head).
struct BlockPos {
    int qb, b, hq;
};
__device__ __forceinline__ BlockPos map_block(int n_qblocks, int batch, int n_heads, int bid) {
    const int BH = batch * n_heads;
    int qb, bh;
    if ((BH & 7) == 0) {
        const int x = bid & 7, j = bid >> 3, hpx = BH >> 3;
        qb = n_qblocks - 1 - j / hpx;
        bh = x * hpx + j % hpx;
    } else {
        qb = n_qblocks - 1 - bid / BH;
        bh = bid % BH;
    }
    return {qb, bh / n_heads, bh % n_heads};
}

// Paired order: workgroup bid owns pair j of one (batch, head), the query
// blocks n_qblocks - 1 - j (item 0) and j (item 1), with the same
// XCD-contiguous (batch, head) ranges as map_block.  With an odd block count
// the middle block forms a pair of its own (item 1 is then skipped).  With at
// most 8 blocks per head (short prompts, where each block's Q/table loads and
// O stores are a large share of its time) every other workgroup on an XCD
// runs its short block first, so that the workgroups' load and store bursts
// do not all meet HBM at once (the 16 x 512-token GQA batch: -4%; the long
// prompt keeps the long block first: +1% the other way).
__device__ __forceinline__ BlockPos map_pair(int n_qblocks, int batch, int n_heads, int bid, int item) {
    const int BH = batch * n_heads;
    int j, bh;
    if ((BH & 7) == 0) {
        const int x = bid & 7, jj = bid >> 3, hpx = BH >> 3;
        j = jj / hpx;
        bh = x * hpx + jj % hpx;
    } else {
        j = bid / BH;
        bh = bid % BH;
    }
    const bool short_first = n_qblocks <= 8 && ((bid >> 3) & 1);
    return {(item == 0) != short_first ? n_qblocks - 1 - j : j, bh / n_heads, bh % n_heads};
}

}  // namespace
}  // namespace pa
