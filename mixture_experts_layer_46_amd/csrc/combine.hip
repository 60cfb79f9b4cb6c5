// Gate-weighted combine back to token order, and router statistics.
//
// Pages cited (by title and section):
//   [FourStage]  "MoE显存与计算开销四阶段手算指南" (bjdmk.com.cn/news/5154310)
//   [Principles] "MoE混合专家模型计算原理与推理部署实战解析" (sheratonhq.com/news/207562)
//
// out[t] = sum_j g[t, j] * y_perm[row_of_pair[t*k + j]]  ([FourStage §2.4]: every token
// sums its k expert outputs weighted by their gates; [Principles §2.2]).  One
// workgroup per token gathers its k grouped rows (16-byte loads, two chunks' worth issued
// before any use), accumulates in fp32 in slot order and rounds once.  Each output row is
// written by exactly one workgroup, so there are no atomics and no ordering races.
// Each grouped row is read once, by its token's workgroup: the loads carry the
// non-temporal hint (fine-grained skewed layer: 0.214 -> 0.195 ms).
#include "common.h"
#include "launch.h"

namespace moe {

// One 16-byte chunk of an output row: the k grouped rows' chunks (already loaded), weighted
// in slot order in fp32, rounded once.
template <bool BF16>
__device__ __forceinline__ uint4 combine_chunk(const uint4 (&v)[8], const int (&rows)[8], const float (&g)[8]) {
    constexpr int NV = BF16 ? 8 : 4;
    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (rows[j] < 0) continue;
        const uint32_t d[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        if constexpr (BF16) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += g[j] * bf16lo_to_f32(d[q]);
                acc[2 * q + 1] += g[j] * bf16hi_to_f32(d[q]);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] += g[j] * __uint_as_float(d[q]);
        }
    }
    uint4 o;
    if constexpr (BF16) {
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
    } else {
        o.x = __float_as_uint(acc[0]);
        o.y = __float_as_uint(acc[1]);
        o.z = __float_as_uint(acc[2]);
        o.w = __float_as_uint(acc[3]);
    }
    return o;
}

__device__ __forceinline__ uint4 load_nt(const uint4* p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}

// Each thread takes two chunks per pass (c and c + 256), so that 2k loads are in flight
// before any use.
template <bool BF16>
__global__ __launch_bounds__(256) void k_combine(const uint4* __restrict__ y,
                                                 const int32_t* __restrict__ row_of_pair,
                                                 const float* __restrict__ w,
                                                 uint4* __restrict__ out, int k, int chunks) {
    const long long t = blockIdx.x;
    int rows[8];
    float g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        rows[j] = (j < k) ? row_of_pair[t * k + j] : -1;
        g[j] = (j < k) ? w[t * k + j] : 0.f;
    }
    for (int c = threadIdx.x; c < chunks; c += 512) {
        const bool two = c + 256 < chunks;
        uint4 v0[8], v1[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (rows[j] >= 0) {
                const uint4* yr = y + (long long)rows[j] * chunks + c;
                v0[j] = load_nt(yr);
                if (two) v1[j] = load_nt(yr + 256);
            }
        out[t * chunks + c] = combine_chunk<BF16>(v0, rows, g);
        if (two) out[t * chunks + c + 256] = combine_chunk<BF16>(v1, rows, g);
    }
}

hipError_t launch_combine(const void* y_perm, const int32_t* row_of_pair, const float* w,
                          void* out, long long T, int k, int H, int dtype, hipStream_t st) {
    if (dtype == MOE_BF16)
        hipLaunchKernelGGL(k_combine<true>, dim3((unsigned)T), dim3(256), 0, st,
                           (const uint4*)y_perm, row_of_pair, w, (uint4*)out, k, H / 8);
    else
        hipLaunchKernelGGL(k_combine<false>, dim3((unsigned)T), dim3(256), 0, st,
                           (const uint4*)y_perm, row_of_pair, w, (uint4*)out, k, H / 4);
    return hipGetLastError();
}

// ------------------------------------------------------------------ router statistics
// One workgroup of 1024 threads (16 wavefronts).  Wavefront w takes tokens w, w+16, ...
// in order; lane l keeps running sums of experts l, l+64, l+128, l+192.  The 16
// partial sums are added in wavefront order, so the result is deterministic.
//   P_e = mean_t softmax(l_t + b)_e          [Principles §4.2]
//   balance = E * sum_e f_e * P_e, f_e = counts[e] / (T*k)
//   entropy = -sum_e f_e ln f_e ; top1 = mean_t max_e softmax(l_t + b)_e
__global__ __launch_bounds__(1024) void k_router_stats(const float* __restrict__ logits,
                                                       const float* __restrict__ bias,
                                                       const int32_t* __restrict__ counts,
                                                       const int32_t* __restrict__ offsets,
                                                       float* __restrict__ stats, long long T,
                                                       int E, int k, int capacity) {
    __shared__ float part[16][256];
    __shared__ float top1[16];
    __shared__ float red[3][256];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
    float t1 = 0.f;
    for (long long t = w; t < T; t += 16) {
        float v[4];
        float m = -INFINITY;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = lane + 64 * q;
            v[q] = (e < E) ? logits[t * E + e] + (bias ? bias[e] : 0.f) : -INFINITY;
            m = fmaxf(m, v[q]);
        }
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        float z = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[q] = (lane + 64 * q < E) ? expf(v[q] - m) : 0.f;
            z += v[q];
        }
        for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
#pragma unroll
        for (int q = 0; q < 4; ++q) sum[q] += v[q] / z;
        t1 += 1.f / z;   // the largest probability is exp(0) / z
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) part[w][lane + 64 * q] = sum[q];
    if (lane == 0) top1[w] = t1;
    __syncthreads();
    const int e = threadIdx.x;
    if (e < 256) {
        float Pe = 0.f;
        for (int i = 0; i < 16; ++i) Pe += part[i][e];
        Pe /= (float)T;
        const float f = (e < E) ? (float)counts[e] / (float)(T * k) : 0.f;
        if (e < E) stats[e] = Pe;
        red[0][e] = (e < E) ? f * Pe : 0.f;
        red[1][e] = (e < E && f > 0.f) ? -f * logf(f) : 0.f;
    }
    __syncthreads();
    for (int off = 128; off >= 1; off >>= 1) {
        if (e < off) {
            red[0][e] += red[0][e + off];
            red[1][e] += red[1][e + off];
        }
        __syncthreads();
    }
    if (e == 0) {
        float s1 = 0.f;
        for (int i = 0; i < 16; ++i) s1 += top1[i];
        stats[E] = (float)E * red[0][0];
        stats[E + 1] = red[1][0];
        stats[E + 2] = s1 / (float)T;
        stats[E + 3] = capacity > 0 ? 1.f - (float)offsets[E] / (float)(T * k) : 0.f;
    }
}

hipError_t launch_router_stats(const float* logits, const float* bias, const int32_t* counts,
                               const int32_t* offsets, float* stats, long long T, int E, int k,
                               int capacity, hipStream_t st) {
    hipLaunchKernelGGL(k_router_stats, dim3(1), dim3(1024), 0, st, logits, bias, counts, offsets,
                       stats, T, E, k, capacity);
    return hipGetLastError();
}

}  // namespace moe
