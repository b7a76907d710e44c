// Decode attention for gfx950 (MI355X): one new token per sequence against
// the KV cache, with RoPE applied to the cached keys inside the kernel.
//
// What is computed: for sequence b whose new token sits at position
// P = pos_offsets[b] (its K/V already written to the cache), every query head
// h attends to the logical keys j = 0 .. P, key j read from cache slot
// kv_map[b][j] and rotated at position j, the query rotated at position P
// ("手写内核实现6倍prefill加速" page, §3.1 RoPE as a complex multiply with
// position-indexed tables; §3.2 keys read through the index map in logical
// order).  The MNN-on-K3 blog (§五, §六) notes that decode attention is a
// short matrix-vector product bound by memory bandwidth, and runs it as
// blocked online softmax; the MI355X design below follows from that:
//
//  * bandwidth first: every cached K and V row is read exactly once per
//    (sequence, KV head) and serves all the query heads that share the KV
//    head (G of them per workgroup);
//  * one key per 16-lane row of a wave (4 keys per wave per step, 16 per
//    workgroup), D/16 elements per lane, fp32 arithmetic on the vector ALUs
//    (the arithmetic intensity is about G flop per byte, far below the
//    matrix-core ridge), dot products reduced across the 16 lanes with DPP;
//  * each 16-lane row keeps its own online-softmax state (running max,
//    running sum, unnormalised O) with the lazy rescale of the prefill
//    kernel; rows, then waves, are merged by the log-sum-exp rule at the end;
//  * long contexts are split over several workgroups (split-K) so that a
//    small batch still fills 256 CUs; the partial (O, max, sum) triples go to
//    a caller-provided workspace and a second small kernel merges them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "internal.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeysPerStep = 4 * kWaves;  // one key per 16-lane row
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kSlack = 8.0f;  // log2 units, as in the prefill kernel
constexpr int kSeg = 2048;      // map entries staged in LDS at a time

// Sum over the 16 lanes of a row; every lane of the row receives the sum.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// N independent sums reduced in lockstep: each DPP step reads a value written
// N instructions earlier, so the steps need no wait states between them (one
// chain at a time, each step waits for the one before).
template <int N>
__device__ __forceinline__ void row_sum16(float (&x)[N]) {
#pragma unroll
    for (int g = 0; g < N; ++g) x[g] += dpp<0xB1>(x[g]);   // quad_perm [1,0,3,2]
#pragma unroll
    for (int g = 0; g < N; ++g) x[g] += dpp<0x4E>(x[g]);   // quad_perm [2,3,0,1]
#pragma unroll
    for (int g = 0; g < N; ++g) x[g] += dpp<0x141>(x[g]);  // row_half_mirror: the other quad of the half row
#pragma unroll
    for (int g = 0; g < N; ++g) x[g] += dpp<0x140>(x[g]);  // row_mirror: the other half of the row
}

// Combine the same lane position of the four 16-lane rows.
__device__ __forceinline__ float rows_max4(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum4(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// exp2(m - M) with an empty state (m = -inf) weighing nothing.
__device__ __forceinline__ float weight(float m, float M) {
    return m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m - M);
}

// E consecutive elements of a row as fp32 (bf16 widened exactly).
template <int E, bool F32>
__device__ __forceinline__ void load_row(const void* base, size_t elem, float* x) {
    if (F32) {
        const float* p = static_cast<const float*>(base) + elem;
#pragma unroll
        for (int e = 0; e < E; e += 2) {
            const float2 t = *reinterpret_cast<const float2*>(p + e);
            x[e] = t.x;
            x[e + 1] = t.y;
        }
    } else {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + elem);
#pragma unroll
        for (int e = 0; e < E; e += 2) {
            const uint32_t w = p[e / 2];
            x[e] = __uint_as_float(w << 16);
            x[e + 1] = __uint_as_float(w & 0xffff0000u);
        }
    }
}

// A row fragment kept as loaded (bf16 pairs stay packed until used).
template <int E, bool F32>
struct Raw {
    static constexpr int N = F32 ? E : E / 2;
    uint32_t w[N];
    __device__ __forceinline__ void load(const void* base, size_t elem) {
        const uint32_t* p = F32 ? reinterpret_cast<const uint32_t*>(static_cast<const float*>(base) + elem)
                                : reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + elem);
#pragma unroll
        for (int i = 0; i < N; i += 2) {
            const uint2 t = *reinterpret_cast<const uint2*>(p + i);
            w[i] = t.x;
            if (i + 1 < N) w[i + 1] = t.y;
        }
    }
    __device__ __forceinline__ float at(int e) const {
        if (F32) return __uint_as_float(w[e]);
        return (e & 1) ? __uint_as_float(w[e / 2] & 0xffff0000u) : __uint_as_float(w[e / 2] << 16);
    }
};

// Rotate E/2 adjacent pairs in place with their (cos, sin) table entries.
template <int E>
__device__ __forceinline__ void rotate(float* x, const float* tab) {
#pragma unroll
    for (int e = 0; e < E; e += 2) {
        const float2 cs = *reinterpret_cast<const float2*>(tab + e);
        const float a = x[e], b = x[e + 1];
        x[e] = fmaf(a, cs.x, -b * cs.y);
        x[e + 1] = fmaf(a, cs.y, b * cs.x);
    }
}

// Workgroup (b, head group, split): keys [lo, hi) of sequence b for the G
// query heads hq0 .. hq0+G-1 (all sharing KV head hq0 / (Hq / Hkv)).
template <int D, int G, bool F32>
__global__ __launch_bounds__(kThreads, G >= 8 ? 2 : 4) void decode_kernel(DecodeArgs a) {
    constexpr int E = D / 16;  // elements per lane
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int row = lane >> 4, sub = lane & 15;
    const int n_groups = a.n_heads / G;
    const int split = blockIdx.x % a.n_split;
    const int grp = (blockIdx.x / a.n_split) % n_groups;
    const int b = blockIdx.x / (a.n_split * n_groups);
    const int hq0 = grp * G;
    const int kvh = hq0 / (a.n_heads / a.n_kv_heads);

    __shared__ float red[kWaves][G][D + 2];
    __shared__ int smap[kSeg];

    const int P = a.pos_offsets ? a.pos_offsets[b] : 0;
    const bool in_range = P >= 0 && static_cast<long long>(P) + 1 <= a.max_seq &&
                          static_cast<long long>(P) + 1 <= a.map_stride;
    const int n_keys = in_range ? P + 1 : 0;
    const int chunk = ((n_keys + a.n_split - 1) / a.n_split + kKeysPerStep - 1) / kKeysPerStep * kKeysPerStep;
    const int lo = min(split * chunk, n_keys), hi = min(lo + chunk, n_keys);
    if (!in_range && split == 0 && threadIdx.x == 0) atomicOr(a.status, 1);

    // Q' of the G heads at position P, pre-scaled for exp2.
    float q[G][E];
    {
        const size_t tab = static_cast<size_t>(in_range ? P : 0) * D + sub * E;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            load_row<E, F32>(a.q, (static_cast<size_t>(b) * a.n_heads + hq0 + g) * D + sub * E, q[g]);
            rotate<E>(q[g], a.rope_f32 + tab);
#pragma unroll
            for (int e = 0; e < E; ++e) q[g][e] *= a.logit_scale;
        }
    }

    float m[G], l[G], acc[G][E];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = kNegInf;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
    }

    const int32_t* map = a.kv_map + static_cast<size_t>(b) * a.map_stride;
    const size_t row_elems = static_cast<size_t>(a.n_kv_heads) * D;
    const size_t head_off = static_cast<size_t>(kvh) * D + sub * E;
    const int my = w * 4 + row;

    // The slots of a segment of keys are staged in LDS first (one coalesced
    // read of the map), so no step waits on a map load before it can address
    // its K/V rows.  Within a segment: two-stage pipeline, the rows of step
    // i+1 are requested before step i is computed.
    for (int s0 = lo; s0 < hi; s0 += kSeg) {
        const int s1 = min(s0 + kSeg, hi);
        __syncthreads();
        for (int i = threadIdx.x; i < s1 - s0; i += kThreads) {
            int sl = map[s0 + i];
            if (static_cast<unsigned>(sl) >= static_cast<unsigned>(a.n_slots)) {
                atomicOr(a.status, 1);
                sl = 0;
            }
            smap[i] = sl;
        }
        __syncthreads();

        // One step: key j of this row from (kc, vc) while the rows of the next
        // step go to (kn, vn).  The loop below runs two steps per iteration
        // with the register sets swapped, so no step copies the next rows.
        auto step = [&](int j0, int j, const Raw<E, F32>& kc, const Raw<E, F32>& vc, Raw<E, F32>& kn,
                        Raw<E, F32>& vn) {
            if (j0 + kKeysPerStep < s1) {
                const size_t r = static_cast<size_t>(smap[min(j + kKeysPerStep, s1 - 1) - s0]) * row_elems + head_off;
                kn.load(a.k, r);
                vn.load(a.v, r);
            }
            const bool valid = j < s1;
            float kx[E];
#pragma unroll
            for (int e = 0; e < E; ++e) kx[e] = kc.at(e);
            rotate<E>(kx, a.rope_f32 + static_cast<size_t>(min(j, s1 - 1)) * D + sub * E);
            float sc[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                sc[g] = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) sc[g] = fmaf(q[g][e], kx[e], sc[g]);
            }
            row_sum16(sc);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const bool need = valid && sc[g] > m[g] + kSlack;
                if (__builtin_amdgcn_ballot_w64(need)) {
                    const float m_new = need ? sc[g] : m[g];
                    const float alpha = weight(m[g], m_new);
                    m[g] = m_new;
                    l[g] *= alpha;
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[g][e] *= alpha;
                }
                const float p = valid ? __builtin_amdgcn_exp2f(sc[g] - m[g]) : 0.f;
                l[g] += p;
#pragma unroll
                for (int e = 0; e < E; ++e) acc[g][e] = fmaf(p, vc.at(e), acc[g][e]);
            }
        };
        Raw<E, F32> k0, v0, k1, v1;
        {
            const size_t r = static_cast<size_t>(smap[min(s0 + my, s1 - 1) - s0]) * row_elems + head_off;
            k0.load(a.k, r);
            v0.load(a.v, r);
        }
        for (int j0 = s0; j0 < s1; j0 += 2 * kKeysPerStep) {
            step(j0, j0 + my, k0, v0, k1, v1);
            if (j0 + kKeysPerStep >= s1) break;
            step(j0 + kKeysPerStep, j0 + kKeysPerStep + my, k1, v1, k0, v0);
        }
    }

    // Merge the four rows of the wave, then the waves (log-sum-exp rule).
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float M = rows_max4(m[g]);
        const float f = weight(m[g], M);
        const float L = rows_sum4(l[g] * f);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] = rows_sum4(acc[g][e] * f);
        if (row == 0) {
#pragma unroll
            for (int e = 0; e < E; ++e) red[w][g][sub * E + e] = acc[g][e];
            if (sub == 0) {
                red[w][g][D] = M;
                red[w][g][D + 1] = L;
            }
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
        const int g = idx / D, d = idx % D;
        float M = kNegInf;
#pragma unroll
        for (int x = 0; x < kWaves; ++x) M = fmaxf(M, red[x][g][D]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int x = 0; x < kWaves; ++x) {
            const float f = weight(red[x][g][D], M);
            L = fmaf(f, red[x][g][D + 1], L);
            O = fmaf(f, red[x][g][d], O);
        }
        const size_t bh = static_cast<size_t>(b) * a.n_heads + hq0 + g;
        if (a.n_split == 1) {
            a.out[bh * D + d] = L > 0.f ? O / L : 0.f;
        } else {
            const size_t part = bh * a.n_split + split;
            a.ws[part * D + d] = O;
            if (d == 0) {
                float* ml = a.ws + static_cast<size_t>(a.batch) * a.n_heads * a.n_split * D;
                ml[2 * part] = M;
                ml[2 * part + 1] = L;
            }
        }
    }
}

// O = sum_s w_s O_s / sum_s w_s l_s with w_s = exp2(m_s - max m), in one
// pass over the splits (running max, rescaled running sums).  The loads of
// four splits are issued together before any of them is used; the O part of
// an empty split (max = -inf) may be unwritten, so it is selected out rather
// than weighted.  One wave per (b, h); lane d handles dims d and d + 64.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
    constexpr int PER = (D + 63) / 64;
    constexpr int CH = 4;  // splits whose loads are in flight together
    const size_t bh = blockIdx.x;
    const float* ml = a.ws + static_cast<size_t>(a.batch) * a.n_heads * a.n_split * D;
    float M = kNegInf, L = 0.f, O[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) O[i] = 0.f;
    for (int s0 = 0; s0 < a.n_split; s0 += CH) {
        float2 st[CH];
        float o[CH][PER];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int s = s0 + c;
            st[c] = make_float2(kNegInf, 0.f);
#pragma unroll
            for (int i = 0; i < PER; ++i) o[c][i] = 0.f;
            if (s < a.n_split) {
                const size_t part = bh * a.n_split + s;
                st[c] = *reinterpret_cast<const float2*>(ml + 2 * part);
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    const int d = threadIdx.x + 64 * i;
                    if (d < D) o[c][i] = a.ws[part * D + d];
                }
            }
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (st[c].x == kNegInf) continue;  // empty split (or past the last)
            const float M2 = fmaxf(M, st[c].x);
            const float f_old = weight(M, M2), f_new = __builtin_amdgcn_exp2f(st[c].x - M2);
            L = L * f_old + st[c].y * f_new;
#pragma unroll
            for (int i = 0; i < PER; ++i) O[i] = O[i] * f_old + o[c][i] * f_new;
            M = M2;
        }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int d = threadIdx.x + 64 * i;
        if (d < D) a.out[bh * D + d] = L > 0.f ? O[i] / L : 0.f;
    }
}

// The same merge for the many short rows of split-K prefill: each thread owns
// 4 dims (16-byte loads and stores) of one row, a workgroup 256 / (D/4) rows.
template <int D>
__global__ __launch_bounds__(256) void split_merge_rows_kernel(DecodeArgs a) {
    constexpr int C4 = D / 4;         // float4 per row
    constexpr int RPB = 256 / C4;     // rows per workgroup
    constexpr int CH = 4;             // splits whose loads are in flight together
    const int r = static_cast<int>(threadIdx.x) / C4, c4 = static_cast<int>(threadIdx.x) % C4;
    const size_t rows = static_cast<size_t>(a.batch) * a.n_heads;
    const size_t row = static_cast<size_t>(blockIdx.x) * RPB + r;
    if (r >= RPB || row >= rows) return;
    const float* ml = a.ws + rows * a.n_split * D;
    float M = kNegInf, L = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < a.n_split; s0 += CH) {
        float2 st[CH];
        float4 o[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int sp = s0 + c;
            st[c] = make_float2(kNegInf, 0.f);
            o[c] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (sp < a.n_split) {
                const size_t part = row * a.n_split + sp;
                st[c] = *reinterpret_cast<const float2*>(ml + 2 * part);
                o[c] = *reinterpret_cast<const float4*>(a.ws + part * D + 4 * c4);
            }
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (st[c].x == kNegInf) continue;  // empty split (its O part may be unwritten) or past the last
            const float M2 = fmaxf(M, st[c].x);
            const float f_old = weight(M, M2), f_new = __builtin_amdgcn_exp2f(st[c].x - M2);
            L = L * f_old + st[c].y * f_new;
            O = make_float4(O.x * f_old + o[c].x * f_new, O.y * f_old + o[c].y * f_new, O.z * f_old + o[c].z * f_new,
                            O.w * f_old + o[c].w * f_new);
            M = M2;
        }
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    *reinterpret_cast<float4*>(a.out + row * D + 4 * c4) = make_float4(O.x * inv, O.y * inv, O.z * inv, O.w * inv);
}

template <int D, int G, bool F32>
hipError_t launch_g(const DecodeArgs& a, hipStream_t s) {
    const long long blocks = static_cast<long long>(a.batch) * (a.n_heads / G) * a.n_split;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_kernel<D, G, F32>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, a);
    if (a.n_split > 1) {
        hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(static_cast<unsigned>(a.batch * a.n_heads)), dim3(64), 0,
                           s, a);
    }
    return hipGetLastError();
}

template <int D, bool F32>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
    switch (decode_group(a.n_heads, a.n_kv_heads)) {
        case 8: return launch_g<D, 8, F32>(a, s);
        case 4: return launch_g<D, 4, F32>(a, s);
        case 2: return launch_g<D, 2, F32>(a, s);
        default: return launch_g<D, 1, F32>(a, s);
    }
}

}  // namespace

int decode_group(int n_heads, int n_kv_heads) {
    const int g = n_heads / n_kv_heads;
    return g % 8 == 0 ? 8 : g % 4 == 0 ? 4 : g % 2 == 0 ? 2 : 1;
}

hipError_t launch_split_merge(int head_dim, const DecodeArgs& a, hipStream_t s) {
    const long long rows = static_cast<long long>(a.batch) * a.n_heads;
    const int rpb = 256 / (head_dim / 4);
    const long long blocks = (rows + rpb - 1) / rpb;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 g(static_cast<unsigned>(blocks));
    switch (head_dim) {
        case 64: hipLaunchKernelGGL((split_merge_rows_kernel<64>), g, dim3(256), 0, s, a); break;
        case 96: hipLaunchKernelGGL((split_merge_rows_kernel<96>), g, dim3(256), 0, s, a); break;
        case 128: hipLaunchKernelGGL((split_merge_rows_kernel<128>), g, dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Scratch of the no-allocation decode entry point: its split partials go here
// instead of into a caller workspace.  Each device that the library runs on
// holds one copy until the process ends; every call on a device shares it.
// Host code never passes `scratch` itself (on the host that name is only a
// stand-in for the symbol): it passes the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(float** ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<float*>(p);
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_decode(int head_dim, bool f32, const DecodeArgs& a, hipStream_t s) {
    switch (head_dim) {
        case 64: return f32 ? launch_d<64, true>(a, s) : launch_d<64, false>(a, s);
        case 96: return f32 ? launch_d<96, true>(a, s) : launch_d<96, false>(a, s);
        case 128: return f32 ? launch_d<128, true>(a, s) : launch_d<128, false>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
