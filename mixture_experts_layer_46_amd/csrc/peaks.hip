// Peak-rate microbenchmarks (dense bf16 MFMA and HBM streaming); declarations, argument
// meaning and errors: include/moe_peaks.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "launch.h"
#include "moe_peaks.h"

namespace moe {
namespace {

// One iteration is the outer product of 4 A and 8 B fragments into 32 independent
// accumulators, as in a GEMM K step: consecutive MFMAs on one accumulator are 32 issues
// apart, far beyond the instruction's latency, so the loop is bound by MFMA issue.
__global__ __launch_bounds__(256, 1) void k_peak_mfma(int iters, float* __restrict__ sink,
                                                     uint64_t* __restrict__ clocks) {
    const int tid = threadIdx.x;
    const uint32_t seed = 0x3f803f80u ^ (uint32_t)(tid * 0x00010001u);
    bf16x8_t a[4], b[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t v = seed ^ (uint32_t)((i + 1) * 0x00400040u);
        a[i] = __builtin_bit_cast(bf16x8_t, u32x4_t{v, v ^ 0x00200020u, v ^ 0x00100010u, v});
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t v = seed ^ (uint32_t)((i + 1) * 0x00080008u);
        b[i] = __builtin_bit_cast(bf16x8_t, u32x4_t{v, v ^ 0x00040004u, v, v ^ 0x00020002u});
    }
    f32x4_t acc[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        // a distinct start value per accumulator (one shared zero register would stop
        // the compiler from updating the accumulators in place)
        acc[c] = f32x4_t{(float)c, 0.f, 0.f, 0.f};
        asm volatile("" : "+a"(acc[c]));
    }
    const uint64_t c0 = clock64(), r0 = wall_clock64();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 32; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j >> 3], b[j & 7], acc[j], 0, 0, 0);
    }
    const uint64_t c1 = clock64(), r1 = wall_clock64();
    float t = 0.f;
#pragma unroll
    for (int c = 0; c < 32; ++c) t += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    sink[(size_t)blockIdx.x * 256 + tid] = t;
    if (blockIdx.x == 0 && tid == 0) {
        clocks[0] = c1 - c0;
        clocks[1] = r1 - r0;
    }
}

constexpr int kUnroll = 4;

template <bool COPY>
__global__ __launch_bounds__(256) void k_peak_stream(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                     size_t n16, float* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * 256;
    uint32_t dig = 0;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride * kUnroll) {
        u32x4_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (i + u * stride < n16) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (i + u * stride < n16) {
                if constexpr (COPY) __builtin_nontemporal_store(v[u], dst + i + u * stride);
                else dig ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
            }
    }
    if constexpr (!COPY) sink[(size_t)blockIdx.x * 256 + threadIdx.x] = (float)dig;
}

bool aligned(const void* p) { return ((uintptr_t)p & 15u) == 0; }

moe_status check_stream(const void* src, const void* dst, bool copy, size_t bytes, int blocks,
                        const float* sink) {
    if (!src) return report_error(MOE_ERR_NULL, "src is NULL");
    if (copy && !dst) return report_error(MOE_ERR_NULL, "dst is NULL");
    if (!copy && !sink) return report_error(MOE_ERR_NULL, "sink is NULL");
    if (bytes == 0 || bytes % 16 != 0) return report_error(MOE_ERR_SHAPE, "bytes must be a positive multiple of 16");
    if (blocks < 1 || blocks > 65536) return report_error(MOE_ERR_SHAPE, "blocks outside [1, 65536]");
    if (!aligned(src) || (copy && !aligned(dst)) || (!copy && !aligned(sink)))
        return report_error(MOE_ERR_ALIGN, "pointers must be 16-byte aligned");
    if (copy) {
        const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
        if (a < b + bytes && b < a + bytes) return report_error(MOE_ERR_SHAPE, "src and dst overlap");
    }
    return MOE_OK;
}

moe_status launch_status(hipError_t e) {
    if (e != hipSuccess) return report_error(MOE_ERR_HIP, hipGetErrorString(e));
    return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_peak_mfma_bf16(int blocks, int iters, float* sink, uint64_t* clocks, int* wall_khz,
                              hipStream_t stream) {
    if (!sink || !clocks) return report_error(MOE_ERR_NULL, "sink and clocks are required");
    if (blocks < 1 || blocks > 65536 || iters < 1) return report_error(MOE_ERR_SHAPE, "blocks outside [1, 65536] or iters < 1");
    if (!aligned(sink) || ((uintptr_t)clocks & 7u) != 0) return report_error(MOE_ERR_ALIGN, "misaligned pointer");
    if (wall_khz) {
        int dev = 0, khz = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
        if (e != hipSuccess) return launch_status(e);
        *wall_khz = khz;
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_peak_mfma, dim3(blocks), dim3(256), 0, stream, iters, sink, clocks);
    return launch_status(hipGetLastError());
}

moe_status moe_peak_hbm_read(const void* src, size_t bytes, int blocks, float* sink, hipStream_t stream) {
    moe_status st = check_stream(src, nullptr, false, bytes, blocks, sink);
    if (st != MOE_OK) return st;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_peak_stream<false>, dim3(blocks), dim3(256), 0, stream, (const u32x4_t*)src,
                       (u32x4_t*)nullptr, bytes / 16, sink);
    return launch_status(hipGetLastError());
}

moe_status moe_peak_hbm_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t stream) {
    moe_status st = check_stream(src, dst, true, bytes, blocks, nullptr);
    if (st != MOE_OK) return st;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_peak_stream<true>, dim3(blocks), dim3(256), 0, stream, (const u32x4_t*)src,
                       (u32x4_t*)dst, bytes / 16, (float*)nullptr);
    return launch_status(hipGetLastError());
}

}  // extern "C"
