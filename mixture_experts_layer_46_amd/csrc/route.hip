// Router: gate projection (fp32) and per-token top-k with renormalised gates.
//
// Pages cited (by title and section):
//   [FourStage]  "MoE显存与计算开销四阶段手算指南" (bjdmk.com.cn/news/5154310)
//   [Principles] "MoE混合专家模型计算原理与推理部署实战解析" (sheratonhq.com/news/207562)
//
// logits = x @ W_g in fp32 ([FourStage §2.1]; [Principles §2.4]: the gate stays fp32 so
// near-equal logits are ranked the same way).  The projection is a thin GEMM
// ([T, H] x [H, E], E <= 256) run on the fp32 MFMA (v_mfma_f32_16x16x4_f32): exact
// widening of bf16 x, fp32 products and accumulation.  Top-k is one wavefront per
// token: each lane holds up to four experts, k rounds of a wave-wide arg-max pick
// the winners ([FourStage §2.2]); gates are the softmax over the chosen logits,
// which equals the full softmax renormalised over the k chosen ([Principles §2.2]).
#include "common.h"
#include "launch.h"

namespace moe {

// ------------------------------------------------------------------ gate projection
// Tile: GT_M tokens x 64 experts per workgroup, K step 32.  Wave w owns expert columns
// [16w, 16w + 16) and all GT_M rows (GT_M / 16 MFMA blocks).
constexpr int GT_E = 64;
constexpr int GT_K = 32;
constexpr int GT_PAD = 16;   // row pad (floats): lane groups of 16 land on distinct banks

template <int GT_M, typename XT>
__global__ __launch_bounds__(256) void k_gate_logits(const XT* __restrict__ x,
                                                     const float* __restrict__ wg,
                                                     float* __restrict__ logits,
                                                     int T, int H, int E) {
    __shared__ float sA[GT_K][GT_M + GT_PAD];   // x tile, k-major
    __shared__ float sB[GT_K][GT_E + GT_PAD];   // W_g tile
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m0 = blockIdx.x * GT_M, e0 = blockIdx.y * GT_E;
    constexpr int FM = GT_M / 16;
    f32x4_t acc[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < H; k0 += GT_K) {
        // x tile: GT_M rows x 32 k, converted to fp32, stored transposed.
        for (int c = tid; c < GT_M * (GT_K / 4); c += 256) {
            const int r = c / (GT_K / 4), kq = (c % (GT_K / 4)) * 4;
            const int t = m0 + r, kk = k0 + kq;
            float v[4] = {0.f, 0.f, 0.f, 0.f};
            if (t < T && kk < H) {   // H % 8 == 0, so a group of 4 never straddles H
                if constexpr (sizeof(XT) == 4) {
                    const float4 q = *reinterpret_cast<const float4*>(x + (size_t)t * H + kk);
                    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
                } else {
                    const uint2 q = *reinterpret_cast<const uint2*>(x + (size_t)t * H + kk);
                    v[0] = bf16lo_to_f32(q.x); v[1] = bf16hi_to_f32(q.x);
                    v[2] = bf16lo_to_f32(q.y); v[3] = bf16hi_to_f32(q.y);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) sA[kq + i][r] = v[i];
        }
        // W_g tile: 32 k x 64 experts (E may be smaller: zero-fill).
        for (int c = tid; c < GT_K * GT_E; c += 256) {
            const int kr = c / GT_E, ec = c % GT_E;
            const int kk = k0 + kr, e = e0 + ec;
            sB[kr][ec] = (kk < H && e < E) ? wg[(size_t)kk * E + e] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < GT_K; ks += 4) {
            const float b = sB[ks + (lane >> 4)][wave * 16 + (lane & 15)];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const float a = sA[ks + (lane >> 4)][fm * 16 + (lane & 15)];
                acc[fm] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[fm], 0, 0, 0);
            }
        }
        __syncthreads();
    }
    // 16x16 fp32 block: lane holds column (lane & 15), rows 4*(lane >> 4) + v.
    const int e = e0 + wave * 16 + (lane & 15);
    if (e < E) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = m0 + fm * 16 + 4 * (lane >> 4) + v;
                if (t < T) logits[(size_t)t * E + e] = acc[fm][v];
            }
    }
}

// ------------------------------------------------------------------------- top-k
struct Cand {
    float s;    // ranking score (l + b)
    float g;    // value the gate is computed from
    int i;      // expert index (>= E: empty)
};

__device__ __forceinline__ bool better(const Cand& a, const Cand& b) {
    // larger score first; equal scores (IEEE ==, so -0 == +0) to the lower index
    return (a.s > b.s) || (a.s == b.s && a.i < b.i);
}

__device__ __forceinline__ Cand wave_best(Cand c) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        Cand o;
        o.s = __shfl_xor(c.s, off);
        o.g = __shfl_xor(c.g, off);
        o.i = __shfl_xor(c.i, off);
        if (o.i < 0x7fffffff && (c.i == 0x7fffffff || better(o, c))) c = o;
    }
    return c;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

// One wavefront per token, four tokens per workgroup.
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits,
                                              const float* __restrict__ bias,
                                              int32_t* __restrict__ topk_idx,
                                              float* __restrict__ topk_w,
                                              long long T, int E, int k, unsigned flags) {
    const int lane = threadIdx.x & 63;
    const long long t = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const bool select_only = flags & MOE_FLAG_BIAS_SELECT_ONLY;
    const bool no_renorm = flags & MOE_FLAG_NO_RENORM;
    float s[4], g[4];
    bool live[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        live[q] = e < E;
        const float l = live[q] ? logits[t * E + e] : 0.f;
        const float b = (live[q] && bias) ? bias[e] : 0.f;
        s[q] = l + b;                       // one fp32 add: the ranking score
        g[q] = select_only ? l : s[q];      // what the gate is computed from
    }
    int sel_i[8];
    float sel_g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        sel_i[j] = 0;
        sel_g[j] = 0.f;
        if (j < k) {
            Cand c{0.f, 0.f, 0x7fffffff};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (!live[q]) continue;
                const Cand o{s[q], g[q], lane + 64 * q};
                if (c.i == 0x7fffffff || better(o, c)) c = o;
            }
            c = wave_best(c);
            sel_i[j] = c.i;
            sel_g[j] = c.g;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (c.i == lane + 64 * q) live[q] = false;
        }
    }
    // gates: exp(g_j - m) / sum, m the largest g among the chosen (slot 0 unless the
    // gate values differ from the ranking scores)
    float m = sel_g[0];
#pragma unroll
    for (int j = 1; j < 8; ++j)
        if (j < k) m = fmaxf(m, sel_g[j]);
    float den = 0.f;
    if (no_renorm) {
        // full softmax over every expert of the token
        float gm = -INFINITY;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (lane + 64 * q < E) gm = fmaxf(gm, g[q]);
        m = wave_max(gm);
        float part = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (lane + 64 * q < E) part += expf(g[q] - m);
        den = wave_sum(part);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < k) den += expf(sel_g[j] - m);
    }
    if (lane < k) {
        float gj = 0.f;
        int ij = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j == lane) { gj = sel_g[j]; ij = sel_i[j]; }
        topk_idx[t * k + lane] = ij;
        topk_w[t * k + lane] = expf(gj - m) / den;
    }
}

// -------------------------------------------------------------------- launchers
hipError_t launch_gate_logits(const void* x, int dtype, const float* wg, float* logits,
                              long long T, int H, int E, hipStream_t st) {
    const dim3 blk(256);
    // 32-token tiles when E fits one 64-expert tile (more workgroups), else 64.
    if (E <= GT_E) {
        const dim3 grid((unsigned)((T + 31) / 32), 1);
        if (dtype == MOE_F32)
            hipLaunchKernelGGL((k_gate_logits<32, float>), grid, blk, 0, st,
                               (const float*)x, wg, logits, (int)T, H, E);
        else
            hipLaunchKernelGGL((k_gate_logits<32, bf16_t>), grid, blk, 0, st,
                               (const bf16_t*)x, wg, logits, (int)T, H, E);
    } else {
        const dim3 grid((unsigned)((T + 63) / 64), (unsigned)((E + GT_E - 1) / GT_E));
        if (dtype == MOE_F32)
            hipLaunchKernelGGL((k_gate_logits<64, float>), grid, blk, 0, st,
                               (const float*)x, wg, logits, (int)T, H, E);
        else
            hipLaunchKernelGGL((k_gate_logits<64, bf16_t>), grid, blk, 0, st,
                               (const bf16_t*)x, wg, logits, (int)T, H, E);
    }
    return hipGetLastError();
}

hipError_t launch_topk(const float* logits, const float* bias, int32_t* idx, float* w,
                       long long T, int E, int k, unsigned flags, hipStream_t st) {
    hipLaunchKernelGGL(k_topk, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st,
                       logits, bias, idx, w, T, E, k, flags);
    return hipGetLastError();
}

}  // namespace moe
