// Router: gate projection (fp32) and per-token top-k with renormalised gates.
//
// Pages cited (by title and section):
//   [FourStage]  "MoE显存与计算开销四阶段手算指南" (bjdmk.com.cn/news/5154310)
//   [Principles] "MoE混合专家模型计算原理与推理部署实战解析" (sheratonhq.com/news/207562)
//
// logits = x @ W_g in fp32 ([FourStage §2.1]; [Principles §2.4]: the gate stays fp32 so
// near-equal logits are ranked the same way).  The projection is a thin GEMM
// ([T, H] x [H, E], E <= 256).  For fp32 x, and for short batches, it runs on the fp32
// MFMA (v_mfma_f32_16x16x4_f32): exact widening of bf16 x, fp32 products and
// accumulation.  For bf16 x it runs on the bf16 MFMA with the weights split exactly
// into three bf16 parts (k_gate_logits_x3): the same fp32 products and accumulation.  Top-k is one wavefront per
// token: each lane holds up to four experts, k rounds of a wave-wide arg-max pick
// the winners ([FourStage §2.2]); gates are the softmax over the chosen logits,
// which equals the full softmax renormalised over the k chosen ([Principles §2.2]).
#include "common.h"
#include "launch.h"

namespace moe {

// ------------------------------------------------------------------ gate projection
// Tile: TM tokens x 64 experts per workgroup, K in steps of 64 over this workgroup's
// K range (split-K: grid.z ranges, partial sums written per range and added in order
// by the top-k kernel).  Wave w owns expert columns [16w, 16w + 16) and all TM rows.
// The next step's x and W_g slabs are loaded into registers while the current step's
// MFMAs run from LDS.
constexpr int GT_E = 64;
constexpr int GT_K = 64;

template <int TM, typename XT>
__global__ __launch_bounds__(256) void k_gate_logits(const XT* __restrict__ x,
                                                     const float* __restrict__ wg,
                                                     float* __restrict__ out, int T, int H, int E,
                                                     int kchunk) {
    __shared__ float sA[GT_K][TM + 16];     // x slab, k-major (fp32)
    __shared__ float sB[GT_K][GT_E + 16];   // W_g slab
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m0 = blockIdx.x * TM, e0 = blockIdx.y * GT_E;
    const int kbeg = blockIdx.z * kchunk, kend = min(H, kbeg + kchunk);
    constexpr int FM = TM / 16;
    // x loader: thread -> (row m = tid % TM, 8-k chunk), TM*8 chunks of 8 per step
    constexpr int XCH = TM * 8 / 256 > 0 ? TM * 8 / 256 : 1;   // chunks per thread
    constexpr bool XPART = TM * 8 < 256;                        // some threads idle
    const int xm = tid % TM, xc0 = tid / TM;
    // W loader: thread -> (k row tid/16 + 16 j, 4 experts (tid % 16) * 4)
    const int wk = tid >> 4, we = (tid & 15) * 4;
    float xr[XCH][8];
    float4 wr[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int j = 0; j < XCH; ++j) {
            const int c = xc0 + j * (256 / TM);
            const int t = m0 + xm, kk = k0 + 8 * c;
            const bool ok = (!XPART || tid < TM * 8) && t < T && kk < kend;
#pragma unroll
            for (int i = 0; i < 8; ++i) xr[j][i] = 0.f;
            if (ok) {
                if constexpr (sizeof(XT) == 4) {
                    const float4 a = *reinterpret_cast<const float4*>(x + (size_t)t * H + kk);
                    const float4 b = *reinterpret_cast<const float4*>(x + (size_t)t * H + kk + 4);
                    xr[j][0] = a.x; xr[j][1] = a.y; xr[j][2] = a.z; xr[j][3] = a.w;
                    xr[j][4] = b.x; xr[j][5] = b.y; xr[j][6] = b.z; xr[j][7] = b.w;
                } else {
                    const uint4 q = *reinterpret_cast<const uint4*>(x + (size_t)t * H + kk);
                    const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        xr[j][2 * i] = bf16lo_to_f32(d[i]);
                        xr[j][2 * i + 1] = bf16hi_to_f32(d[i]);
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kk = k0 + wk + 16 * j, e = e0 + we;
            wr[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (kk < kend) {
                if (e + 3 < E) {
                    wr[j] = *reinterpret_cast<const float4*>(wg + (size_t)kk * E + e);
                } else {
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = (e + i < E) ? wg[(size_t)kk * E + e + i] : 0.f;
                    wr[j] = make_float4(v[0], v[1], v[2], v[3]);
                }
            }
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int j = 0; j < XCH; ++j) {
            const int c = xc0 + j * (256 / TM);
            if (!XPART || tid < TM * 8)
#pragma unroll
                for (int i = 0; i < 8; ++i) sA[8 * c + i][xm] = xr[j][i];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<float4*>(&sB[wk + 16 * j][we]) = wr[j];
    };
    f32x4_t acc[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (kbeg < kend) {
        gload(kbeg);
        for (int k0 = kbeg; k0 < kend; k0 += GT_K) {
            __syncthreads();
            lstore();
            __syncthreads();
            if (k0 + GT_K < kend) gload(k0 + GT_K);
#pragma unroll
            for (int ks = 0; ks < GT_K; ks += 4) {
                const float bv = sB[ks + (lane >> 4)][wave * 16 + (lane & 15)];
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const float av = sA[ks + (lane >> 4)][fm * 16 + (lane & 15)];
                    acc[fm] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[fm], 0, 0, 0);
                }
            }
        }
    }
    // 16x16 fp32 block: lane holds column (lane & 15), rows 4*(lane >> 4) + v.
    float* o = out + (size_t)blockIdx.z * T * E;
    const int e = e0 + wave * 16 + (lane & 15);
    if (e < E) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = m0 + fm * 16 + 4 * (lane >> 4) + v;
                if (t < T) o[(size_t)t * E + e] = acc[fm][v];
            }
    }
}

// Gate projection for bf16 x on the bf16 MFMA.  Each fp32 gate weight is split exactly
// into three bf16 parts, w = w1 + w2 + w3 (w1 = bf16(w), w2 = bf16(w - w1), w3 =
// bf16(w - w1 - w2); each difference is exact, and 3 x 8 significant bits cover fp32's
// 24).  A bf16 x times a bf16 part is exact in fp32, so x . w = x . w3 + x . w2 + x . w1
// runs as three v_mfma_f32_16x16x32_bf16 with fp32 accumulation: the same fp32
// products and accumulation as the fp32 MFMA, at 3 x 16 instead of 8 x 32 cycles per
// 32 of K.  (Outside the exact range: weights above about 3.39e38, whose bf16 rounding
// is infinite, and below about 2^-110, whose third part loses low bits.)
// Tile: TM tokens x 64 experts per workgroup, K in steps of 64 over this workgroup's K
// range (split-K as in k_gate_logits).  Wave w owns expert columns [16w, 16w + 16).
// x stays row-major in LDS, the split weights are stored expert-major (k contiguous), so
// both MFMA operands are single 16-byte LDS reads.
__device__ __forceinline__ void split3_bf16(float w, float& h, float& m, float& l) {
    h = (float)(__bf16)w;
    const float r = w - h;
    m = (float)(__bf16)r;
    l = r - m;                   // exactly representable in bf16
}

constexpr int GX_PITCH = GT_K + 8;          // bf16 per LDS row (16-byte pad)

template <int TM>
__global__ __launch_bounds__(256) void k_gate_logits_x3(const bf16_t* __restrict__ x,
                                                        const float* __restrict__ wg,
                                                        float* __restrict__ out, int T, int H, int E,
                                                        int kchunk) {
    __shared__ __attribute__((aligned(16))) bf16_t sX[TM][GX_PITCH];
    __shared__ __attribute__((aligned(16))) bf16_t sW[3][GT_E][GX_PITCH];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m0 = blockIdx.x * TM, e0 = blockIdx.y * GT_E;
    const int kbeg = blockIdx.z * kchunk, kend = min(H, kbeg + kchunk);
    constexpr int FM = TM / 16;
    // x loader: TM rows x 8 chunks of 8 bf16 per step; thread -> (row, XCH chunks)
    constexpr int XCH = TM * 8 / 256 > 0 ? TM * 8 / 256 : 1;
    constexpr bool XPART = TM * 8 < 256;
    const int xrow = tid / (8 / XCH), xc0 = (tid % (8 / XCH)) * XCH;
    // W loader: thread -> k rows 4 kq .. 4 kq + 3, experts 4 eg .. 4 eg + 3
    const int kq = tid & 15, eg = tid >> 4;
    // one K step's operands in registers; two are in flight (the loads of step k + 2 are
    // issued before step k's MFMAs), which covers HBM latency for x
    struct Stage {
        uint4 xr[XCH];
        float4 wr[4];
    };
    auto gload = [&](Stage& sg, int k0) {
#pragma unroll
        for (int j = 0; j < XCH; ++j) {
            const int t = m0 + xrow, kk = k0 + 8 * (xc0 + j);
            sg.xr[j] = make_uint4(0u, 0u, 0u, 0u);
            if ((!XPART || tid < TM * 8) && t < T && kk < kend)
                sg.xr[j] = *reinterpret_cast<const uint4*>(x + (size_t)t * H + kk);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kk = k0 + 4 * kq + j, e = e0 + 4 * eg;
            sg.wr[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (kk < kend) {
                if (e + 3 < E) {
                    sg.wr[j] = *reinterpret_cast<const float4*>(wg + (size_t)kk * E + e);
                } else {
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = (e + i < E) ? wg[(size_t)kk * E + e + i] : 0.f;
                    sg.wr[j] = make_float4(v[0], v[1], v[2], v[3]);
                }
            }
        }
    };
    auto lstore = [&](const Stage& sg) {
        if (!XPART || tid < TM * 8) {
#pragma unroll
            for (int j = 0; j < XCH; ++j) *reinterpret_cast<uint4*>(&sX[xrow][8 * (xc0 + j)]) = sg.xr[j];
        }
        // expert i of this thread: its 4 k values, split into the three bf16 planes
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4* wr = sg.wr;
            const float w4[4] = {i == 0 ? wr[0].x : i == 1 ? wr[0].y : i == 2 ? wr[0].z : wr[0].w,
                                 i == 0 ? wr[1].x : i == 1 ? wr[1].y : i == 2 ? wr[1].z : wr[1].w,
                                 i == 0 ? wr[2].x : i == 1 ? wr[2].y : i == 2 ? wr[2].z : wr[2].w,
                                 i == 0 ? wr[3].x : i == 1 ? wr[3].y : i == 2 ? wr[3].z : wr[3].w};
            float h[4], m[4], l[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) split3_bf16(w4[j], h[j], m[j], l[j]);
            const int e = 4 * eg + i;
            *reinterpret_cast<uint2*>(&sW[0][e][4 * kq]) = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
            *reinterpret_cast<uint2*>(&sW[1][e][4 * kq]) = make_uint2(pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]));
            *reinterpret_cast<uint2*>(&sW[2][e][4 * kq]) = make_uint2(pack_bf16x2(l[0], l[1]), pack_bf16x2(l[2], l[3]));
        }
    };
    f32x4_t acc[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int fr = lane & 15, fq = lane >> 4;
    auto mfma_step = [&]() {
#pragma unroll
        for (int ks = 0; ks < GT_K; ks += 32) {
            bf16x8_t b[3];
#pragma unroll
            for (int p = 0; p < 3; ++p)
                b[p] = *reinterpret_cast<const bf16x8_t*>(&sW[p][16 * wave + fr][ks + 8 * fq]);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&sX[16 * fm + fr][ks + 8 * fq]);
                // the small parts first
                acc[fm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[2], acc[fm], 0, 0, 0);
                acc[fm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[1], acc[fm], 0, 0, 0);
                acc[fm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[0], acc[fm], 0, 0, 0);
            }
        }
    };
    if (kbeg < kend) {
        Stage s0, s1;
        gload(s0, kbeg);
        gload(s1, kbeg + GT_K);                 // (past kend: zeros, no loads)
        for (int k0 = kbeg; k0 < kend; k0 += 2 * GT_K) {
            __syncthreads();
            lstore(s0);
            __syncthreads();
            gload(s0, k0 + 2 * GT_K);
            mfma_step();
            if (k0 + GT_K >= kend) break;
            __syncthreads();
            lstore(s1);
            __syncthreads();
            gload(s1, k0 + 3 * GT_K);
            mfma_step();
        }
    }
    // 16x16 block: lane holds column (lane & 15), rows 4*(lane >> 4) + v.
    float* o = out + (size_t)blockIdx.z * T * E;
    const int e = e0 + wave * 16 + (lane & 15);
    if (e < E) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = m0 + fm * 16 + 4 * (lane >> 4) + v;
                if (t < T) o[(size_t)t * E + e] = acc[fm][v];
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
// `logits` holds `nparts` partial sums [nparts][T][E] (split K); they are added in
// order and, when `logits_out` is given, the sum is written there.
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int nparts,
                                              float* __restrict__ logits_out,
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
        float l = 0.f;
        if (live[q]) {
            l = logits[t * E + e];
            for (int p = 1; p < nparts; ++p) l += logits[(long long)p * T * E + t * E + e];
            if (logits_out) logits_out[t * E + e] = l;
        }
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
// Row-tile height of the gate projection: 16 tokens for short batches (fp32 MFMA), else
// 128 for bf16 x (split weights, whose conversion each workgroup repeats: taller tiles
// amortise it) and 64 for fp32 x.
int gate_tile_rows(long long T, int dtype) { return T <= 256 ? 16 : (dtype == MOE_F32 ? 64 : 128); }

int gate_splits(long long T, int H, int E, int dtype) {
    if (T <= 0) return 1;
    const long long tm = gate_tile_rows(T, dtype);
    const long long base = ((T + tm - 1) / tm) * ((E + GT_E - 1) / GT_E);
    long long sp = (512 + base - 1) / base;
    const long long maxs = (H + 255) / 256;
    if (sp > maxs) sp = maxs;
    return (int)(sp < 1 ? 1 : sp);
}

hipError_t launch_gate_logits(const void* x, int dtype, const float* wg, float* out, long long T, int H,
                              int E, int splits, hipStream_t st) {
    const dim3 blk(256);
    const int kchunk = ((H + splits - 1) / splits + GT_K - 1) / GT_K * GT_K;
    const unsigned gy = (unsigned)((E + GT_E - 1) / GT_E);
    if (T <= 256) {
        const dim3 grid((unsigned)((T + 15) / 16), gy, (unsigned)splits);
        if (dtype == MOE_F32)
            hipLaunchKernelGGL((k_gate_logits<16, float>), grid, blk, 0, st, (const float*)x, wg, out, (int)T, H, E, kchunk);
        else
            hipLaunchKernelGGL((k_gate_logits<16, bf16_t>), grid, blk, 0, st, (const bf16_t*)x, wg, out, (int)T, H, E, kchunk);
    } else if (dtype == MOE_F32) {
        const dim3 grid((unsigned)((T + 63) / 64), gy, (unsigned)splits);
        hipLaunchKernelGGL((k_gate_logits<64, float>), grid, blk, 0, st, (const float*)x, wg, out, (int)T, H, E, kchunk);
    } else {
        const dim3 grid((unsigned)((T + 127) / 128), gy, (unsigned)splits);
        hipLaunchKernelGGL((k_gate_logits_x3<128>), grid, blk, 0, st, (const bf16_t*)x, wg, out, (int)T, H, E, kchunk);
    }
    return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int nparts, float* logits_out, const float* bias, int32_t* idx,
                       float* w, long long T, int E, int k, unsigned flags, hipStream_t st) {
    hipLaunchKernelGGL(k_topk, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st,
                       logits, nparts, logits_out, bias, idx, w, T, E, k, flags);
    return hipGetLastError();
}

}  // namespace moe
