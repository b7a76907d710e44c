// Matrix-core peak and shader clock of the current device, measured: the
// roofline denominators the bench reports next to the vendor figures (the
// XNet-DNN article, §三, measures its GPUs with a micro-benchmark suite and
// plots the kernels against the measured roofline, Fig. 5).
//
// One workgroup of eight waves per CU (two waves per SIMD; an LDS reservation
// keeps a second workgroup off every CU, so each CU holds exactly one), every
// wave issuing nothing but v_mfma_f32_32x32x16_f16 on four independent
// accumulators, so the matrix pipes never wait on a dependency, and operands
// that differ lane by lane (the switching activity, hence the power and the
// clock the chip holds, of real data rather than of constants).  The rate is
// the launch's FLOP over its event-timed wall time (a loop of some 10 ms, so
// the launch itself is noise).  Each workgroup also reads the shader-clock
// counter (s_memtime) and the real-time counter (s_memrealtime, 100 MHz
// nominal) around its loop; the shader clock is their ratio times 100 MHz.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <vector>

#include "device_common.h"
#include "internal.h"

namespace pa {
namespace {

constexpr int kPeakThreads = 512;
constexpr int kReserveLds = 96 * 1024;  // more than half the CU's LDS: one workgroup per CU
constexpr double kRealtimeHz = 100e6;  // nominal rate of s_memrealtime

__global__ __launch_bounds__(kPeakThreads, 1) void mfma_peak_kernel(int iters, float* sink,
                                                                    unsigned long long* ticks) {
    __shared__ float reserve[kReserveLds / sizeof(float)];
    const int lane = threadIdx.x & 63;
    reserve[threadIdx.x] = static_cast<float>(lane);
    f16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = static_cast<_Float16>(0.001f * (lane + i));
        b[i] = static_cast<_Float16>(0.002f * (lane - i));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    __syncthreads();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float acc = reserve[(threadIdx.x + 1) % kPeakThreads];
#pragma unroll
    for (int v = 0; v < 16; ++v) acc += c0[v] + c1[v] + c2[v] + c3[v];
    if (acc == 1234.5f) sink[blockIdx.x * kPeakThreads + threadIdx.x] = acc;  // keeps the loop alive
    if (threadIdx.x == 0) {
        ticks[2 * blockIdx.x] = t1 - t0;
        ticks[2 * blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace

hipError_t measure_device_peak(int iters, double* tflops, double* clock_ghz, hipStream_t s) {
    const int n_wg = device_cus();
    float* sink = nullptr;
    unsigned long long* cyc = nullptr;
    hipError_t e = hipMalloc(&sink, sizeof(float) * static_cast<size_t>(n_wg) * kPeakThreads);
    if (e != hipSuccess) return e;
    e = hipMalloc(&cyc, 2 * sizeof(unsigned long long) * n_wg);
    if (e != hipSuccess) {
        (void)hipFree(sink);
        return e;
    }
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    if ((e = hipEventCreate(&ev0)) == hipSuccess && (e = hipEventCreate(&ev1)) == hipSuccess) {
        // warm-up launch (clocks ramp up), then the timed one
        hipLaunchKernelGGL(mfma_peak_kernel, dim3(n_wg), dim3(kPeakThreads), 0, s, iters / 4 + 1, sink, cyc);
        (void)hipEventRecord(ev0, s);
        hipLaunchKernelGGL(mfma_peak_kernel, dim3(n_wg), dim3(kPeakThreads), 0, s, iters, sink, cyc);
        (void)hipEventRecord(ev1, s);
        e = hipGetLastError();
        if (e == hipSuccess) e = hipEventSynchronize(ev1);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev0, ev1);
        std::vector<unsigned long long> host(2 * n_wg);
        if (e == hipSuccess)
            e = hipMemcpy(host.data(), cyc, 2 * sizeof(unsigned long long) * n_wg, hipMemcpyDeviceToHost);
        if (e == hipSuccess && ms > 0.f) {
            double clk = 0.0, rt = 0.0;
            for (int i = 0; i < n_wg; ++i) {
                clk += static_cast<double>(host[2 * i]);
                rt += static_cast<double>(host[2 * i + 1]);
            }
            const double flop = 2.0 * 32 * 32 * 16 * 4.0 * iters * (kPeakThreads / 64) * static_cast<double>(n_wg);
            *tflops = flop / (ms * 1e-3) / 1e12;
            *clock_ghz = rt > 0.0 ? clk / rt * kRealtimeHz / 1e9 : 0.0;
        }
    }
    if (ev0) (void)hipEventDestroy(ev0);
    if (ev1) (void)hipEventDestroy(ev1);
    (void)hipFree(sink);
    (void)hipFree(cyc);
    return e;
}

}  // namespace pa
