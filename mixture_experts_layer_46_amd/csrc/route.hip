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
// into three bf16 parts (k_gate_logits_x3): the same fp32 products and accumulation.
// Top-k takes 16 lanes per token, each holding up to 16 experts; k rounds of a row-wide
// arg-max pick the winners ([FourStage §2.2]); gates are the softmax over the chosen
// logits, which equals the full softmax renormalised over the k chosen ([Principles §2.2]).
#include <type_traits>

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
__device__ __forceinline__ void split3_bf16(float w, float& h, float& m, float& l) {
    h = (float)(__bf16)w;
    const float r = w - h;
    m = (float)(__bf16)r;
    l = r - m;                   // exactly representable in bf16
}

constexpr int GX_PITCH = GT_K + 8;          // bf16 per LDS row (16-byte pad)

// Tile: 256 tokens x TE experts per workgroup of 8 wavefronts (TE = 128 when E > 64,
// else 64), K in steps of 64 over this workgroup's K range (split-K as in k_gate_logits).
// The wavefronts form a 4 x 2 grid: wavefront (wm, wn) owns tokens [64 wm, 64 wm + 64)
// and experts [wn TE/2, (wn + 1) TE/2), i.e. 4 x TE/32 blocks of 16 x 16 fp32
// accumulators, two wavefronts per SIMD so that one's LDS reads overlap the other's
// MFMAs.  Against a 128-token x 64-expert tile this reads W_g half as often (once per 256
// tokens), and x half as often when E > 64 (once per 128 experts).  The next step's x and
// W_g travel into registers while the current step's MFMAs run from LDS.
template <int TE>
__global__ __launch_bounds__(512, 1) void k_gate_logits_x3(const bf16_t* __restrict__ x,
                                                           const float* __restrict__ wg,
                                                           float* __restrict__ out, int T, int H, int E,
                                                           int kchunk) {
    constexpr int TM = 256;
    constexpr int NB = TE / 32;                 // 16-expert column blocks per wavefront
    constexpr int FM = 4;                       // 16-token row blocks per wavefront
    constexpr int NPAIR = 16 * (TE / 4);        // (k quad, expert quad) pairs of one W step
    __shared__ __attribute__((aligned(16))) bf16_t sX[TM][GX_PITCH];
    __shared__ __attribute__((aligned(16))) bf16_t sW[3][TE][GX_PITCH];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.x * TM, e0 = blockIdx.y * TE;
    const int kbeg = blockIdx.z * kchunk, kend = min(H, kbeg + kchunk);
    // x loader: load i of thread t moves 16 bytes (8 k) of row (t >> 3) + 64 i, chunk t & 7,
    // so the 8 lanes of one row read its 128 bytes of the step together
    const int xr0 = tid >> 3, xc = tid & 7;
    // W loader: thread t < NPAIR takes expert quad eg = t % (TE/4) and k quad kq = t / (TE/4):
    // four float4 rows of 4 experts, so each expert's 4 k values pack into one 8-byte LDS
    // store per plane
    const bool wthr = tid < NPAIR;
    const int eg = tid % (TE / 4), kq = tid / (TE / 4);
    uint4 xr[4];
    float4 wr[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = m0 + xr0 + 64 * i, kk = k0 + 8 * xc;
            xr[i] = make_uint4(0u, 0u, 0u, 0u);
            if (t < T && kk < kend) xr[i] = *reinterpret_cast<const uint4*>(x + (size_t)t * H + kk);
        }
        const int e = e0 + 4 * eg;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int kk = k0 + 4 * kq + r;
            wr[r] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (wthr && kk < kend) {
                if (e + 3 < E) {
                    wr[r] = *reinterpret_cast<const float4*>(wg + (size_t)kk * E + e);
                } else {
                    float v[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) v[c] = (e + c < E) ? wg[(size_t)kk * E + e + c] : 0.f;
                    wr[r] = make_float4(v[0], v[1], v[2], v[3]);
                }
            }
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&sX[xr0 + 64 * i][8 * xc]) = xr[i];
        if (wthr) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {      // expert 4 eg + c: its 4 k values, split in 3 planes
                float h[4], m[4], l[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float4& v = wr[r];
                    split3_bf16(c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w, h[r], m[r], l[r]);
                }
                const int e = 4 * eg + c;
                *reinterpret_cast<uint2*>(&sW[0][e][4 * kq]) = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
                *reinterpret_cast<uint2*>(&sW[1][e][4 * kq]) = make_uint2(pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]));
                *reinterpret_cast<uint2*>(&sW[2][e][4 * kq]) = make_uint2(pack_bf16x2(l[0], l[1]), pack_bf16x2(l[2], l[3]));
            }
        }
    };
    f32x4_t acc[FM][NB];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int fr = lane & 15, fq = lane >> 4;
    if (kbeg < kend) {
        gload(kbeg);
        for (int k0 = kbeg; k0 < kend; k0 += GT_K) {
            __syncthreads();
            lstore();
            __syncthreads();
            if (k0 + GT_K < kend) gload(k0 + GT_K);
#pragma unroll
            for (int ks = 0; ks < GT_K; ks += 32) {
                bf16x8_t b[NB][3], a[FM];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int p = 0; p < 3; ++p)
                        b[nb][p] = *reinterpret_cast<const bf16x8_t*>(
                            &sW[p][wn * (TE / 2) + 16 * nb + fr][ks + 8 * fq]);
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    a[fm] = *reinterpret_cast<const bf16x8_t*>(&sX[64 * wm + 16 * fm + fr][ks + 8 * fq]);
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        // the small parts first
                        acc[fm][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], b[nb][2], acc[fm][nb], 0, 0, 0);
                        acc[fm][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], b[nb][1], acc[fm][nb], 0, 0, 0);
                        acc[fm][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], b[nb][0], acc[fm][nb], 0, 0, 0);
                    }
            }
        }
    }
    // 16x16 block: lane holds column (lane & 15), rows 4*(lane >> 4) + v.
    float* o = out + (size_t)blockIdx.z * T * E;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int e = e0 + wn * (TE / 2) + 16 * nb + fr;
        if (e >= E) continue;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = m0 + 64 * wm + fm * 16 + 4 * fq + v;
                if (t < T) o[(size_t)t * E + e] = acc[fm][nb][v];
            }
    }
}

// W_g [H, E] fp32 -> three bf16 planes with w = p0 + p1 + p2 exactly (split3_bf16), once
// per call, so that the gate projection's workgroups copy runs of k instead of splitting
// and transposing weights each.  Layout K-step-major, [H/32][3][E][32]: the 32 k of one
// step of plane p and expert e are 64 contiguous bytes, and one step of one plane for 16
// consecutive experts is 1 KB contiguous, so each direct-to-LDS load of the gate covers
// whole cache lines.  Entries for k >= H (the last step's padding) are never written or read.
// Tile: 64 k x 64 experts through LDS (loads coalesced along E, stores along k).
__global__ __launch_bounds__(256) void k_gate_split_planes(const float* __restrict__ wg, bf16_t* __restrict__ planes,
                                                           int H, int E) {
    __shared__ float tile[64][65];
    const int k0 = blockIdx.x * 64, e0 = blockIdx.y * 64, tid = threadIdx.x;
    if ((E & 3) == 0 && ((uintptr_t)wg & 15) == 0) {   // whole 16-byte runs: 4 loads per thread
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = tid + 256 * u, r = i >> 4, c = 4 * (i & 15);
            const int k = k0 + r, e = e0 + c;
            v[u] = (k < H && e < E) ? *reinterpret_cast<const float4*>(wg + (size_t)k * E + e)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = tid + 256 * u, r = i >> 4, c = 4 * (i & 15);
            tile[r][c] = v[u].x;
            tile[r][c + 1] = v[u].y;
            tile[r][c + 2] = v[u].z;
            tile[r][c + 3] = v[u].w;
        }
    } else {
        for (int i = tid; i < 64 * 64; i += 256) {
            const int r = i >> 6, c = i & 63;
            const int k = k0 + r, e = e0 + c;
            tile[r][c] = (k < H && e < E) ? wg[(size_t)k * E + e] : 0.f;
        }
    }
    __syncthreads();
    for (int i = tid; i < 64 * 8; i += 256) {
        const int c = i >> 3, kq = i & 7;          // expert e0 + c, k run k0 + 8 kq .. + 7
        const int e = e0 + c, k = k0 + 8 * kq;
        if (e >= E || k >= H) continue;            // H % 8 == 0: a run is all inside or all outside
        float h[8], m[8], l[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) split3_bf16(tile[8 * kq + j][c], h[j], m[j], l[j]);
        const uint4 vh = make_uint4(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]), pack_bf16x2(h[4], h[5]),
                                    pack_bf16x2(h[6], h[7]));
        const uint4 vm = make_uint4(pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]), pack_bf16x2(m[4], m[5]),
                                    pack_bf16x2(m[6], m[7]));
        const uint4 vl = make_uint4(pack_bf16x2(l[0], l[1]), pack_bf16x2(l[2], l[3]), pack_bf16x2(l[4], l[5]),
                                    pack_bf16x2(l[6], l[7]));
        // K step ks = k / 32 of plane p, expert e at ((ks * 3 + p) * E + e) * 32 + k % 32
        const size_t base = ((size_t)(k >> 5) * 3 * E + e) * 32 + (k & 31);
        *reinterpret_cast<uint4*>(planes + base) = vh;
        *reinterpret_cast<uint4*>(planes + base + (size_t)E * 32) = vm;
        *reinterpret_cast<uint4*>(planes + base + (size_t)2 * E * 32) = vl;
    }
}

// The gate projection from the pre-split planes, with its operands streamed into LDS by
// direct-to-LDS buffer loads (no register staging: a register stage covered one 64-K step
// of MFMAs against a load latency about twice as long).  Tile: 256 tokens x TE experts,
// eight wavefronts in a 4 x 2 grid (64 tokens x TE/2 experts each, two per SIMD), K steps
// of 32.  A stage holds x (256 rows of 64 bytes) and the three planes (3 TE rows of 64
// bytes), rows swizzled with swa4 for the fragment reads.  The fragments of a step are
// read into registers (two sets, alternating) a step ahead, so a stage is free once they
// are: GS_NS stages hold the DMA of the next GS_NS steps, with one barrier per step in
// the middle of its MFMAs.  Every step issues the same DMA (steps past the K range load
// zeros into a stage nobody reads), so each wavefront waits with a constant count.  MFMA
// order per step and 16-expert block: the plane of the smallest parts first.
constexpr int GS_NS = 4;

// keeps an accumulator in AGPRs (the MFMA then accumulates in place)
__device__ __forceinline__ void gs_pin_acc(f32x4_t& a) { asm volatile("" : "+a"(a)); }
// one 16-byte-per-lane direct-to-LDS load (1 KB per wavefront) at dst
__device__ __forceinline__ void gs_dma(__amdgpu_buffer_rsrc_t r, lds_char* dst, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, off, 0, 0, 0);
}
// no instruction moves across this point (the MFMAs only touch registers, so the barrier's
// memory clobber alone would let the scheduler hoist them above it)
__device__ __forceinline__ void gs_sched_fence() { __builtin_amdgcn_sched_barrier(0); }
// this wavefront's fragment reads are done, then every wavefront's (a bare s_barrier: the
// fence of __syncthreads would also wait for the DMA in flight)
__device__ __forceinline__ void gs_step_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");
}

template <int TE>
struct GateStage {
    static constexpr int TM = 256, BK = 32;
    static constexpr int X_BYTES = TM * BK * 2;              // 16 KB
    static constexpr int W_BYTES = 3 * TE * BK * 2;          // 24 KB (TE 128) or 12 KB
    static constexpr int BYTES = X_BYTES + W_BYTES;
    static constexpr int NI = BYTES / 1024;                  // 1 KB DMA instructions per stage
    static constexpr int DPW_HI = (NI + 7) / 8, DPW_LO = NI / 8;   // per wavefront
    static constexpr int LDS = GS_NS * BYTES;
    static_assert(LDS <= 160 * 1024, "the stages fit the LDS");
    static_assert(NI % 8 == 0 || DPW_HI == DPW_LO + 1, "two DMA counts at most");
};

template <int TE>
__global__ __launch_bounds__(512, 1) void k_gate_logits_p3(const bf16_t* __restrict__ x,
                                                           const bf16_t* __restrict__ planes,
                                                           float* __restrict__ out, int T, int H, int E,
                                                           int kchunk) {
    using S = GateStage<TE>;
    constexpr int TM = S::TM, BK = S::BK, NI = S::NI;
    constexpr int NB = TE / 32;                 // 16-expert column blocks per wavefront
    constexpr int FM = 4;                       // 16-token row blocks per wavefront
    constexpr int DMAX = S::DPW_HI;
    extern __shared__ uint4 gsmem[];
    lds_char* lds = (lds_char*)gsmem;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.x * TM, e0 = blockIdx.y * TE;
    const int kbeg = blockIdx.z * kchunk, kend = min(H, kbeg + kchunk);
    const int KT = kbeg < kend ? (kend - kbeg + BK - 1) / BK : 0;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)((size_t)T * H * 2));
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(planes, (uint32_t)((size_t)3 * E * gate_plane_k(H) * 2));
    // this wavefront's DMA instructions j = wave + 8 i (j < NI): x rows 16 j .. 16 j + 15
    // for j < 16, else plane rows 16 (j - 16) ..; each lane moves one 16-byte chunk
    uint32_t off[DMAX], kq[DMAX];
    bool isx[DMAX];
#pragma unroll
    for (int i = 0; i < DMAX; ++i) {
        const int j = wave + 8 * i;
        isx[i] = j < 16;
        off[i] = kOOB;
        kq[i] = 0;
        if (j < NI) {
            const int r = (isx[i] ? j : j - 16) * 16 + (lane >> 2);   // row in the x or plane region
            const int q = (lane & 3) ^ swa4(r);
            kq[i] = (uint32_t)(kbeg + 8 * q);
            if (isx[i]) {
                const int t = m0 + r;
                if (t < T) off[i] = (uint32_t)(((size_t)t * H + kbeg + 8 * q) * 2);
            } else {
                const int pl = r / TE, e = e0 + r % TE;
                if (e < E) off[i] = (uint32_t)(((((size_t)(kbeg >> 5) * 3 + pl) * E + e) * 32 + 8 * q) * 2);
            }
        }
    }
    auto dma = [&](int step) {                  // the DMA of K step `step` into its stage
        lds_char* st = lds + (step % GS_NS) * S::BYTES;
#pragma unroll
        for (int i = 0; i < DMAX; ++i) {
            const int j = wave + 8 * i;
            if (j < NI) {
                const uint32_t dk = (uint32_t)step * BK;
                // a K step advances x rows by 64 bytes and the planes by one step block
                const uint32_t adv = isx[i] ? (uint32_t)BK * 2 : (uint32_t)(3 * E * BK * 2);
                const uint32_t o = (off[i] != kOOB && step < KT && kq[i] + dk < (uint32_t)kend) ? off[i] + (uint32_t)step * adv : kOOB;
                gs_dma(isx[i] ? rx : rp, st + j * 1024, o);
            }
        }
    };
    // every DMA this wavefront issued has landed except the last `ahead` steps' (which may
    // still be in flight)
    auto wait_dma = [&](auto ahead_c) {
        constexpr int AH = decltype(ahead_c)::value;
        if (NI % 8 == 0 || wave < NI % 8) wait_vmcnt<S::DPW_HI * AH>();
        else wait_vmcnt<S::DPW_LO * AH>();
    };
    f32x4_t acc[FM][NB];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            gs_pin_acc(acc[i][j]);
        }
    const int fr = lane & 15, fq = lane >> 4;
    // fragment read offsets within a stage
    int a_rd[FM], b_rd[NB];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int r = 64 * wm + 16 * fm + fr;
        a_rd[fm] = r * 64 + ((fq ^ swa4(r)) << 4);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int r = wn * (TE / 2) + 16 * nb + fr;
        b_rd[nb] = S::X_BYTES + r * 64 + ((fq ^ swa4(r)) << 4);
    }
    using LdsFrag = const __attribute__((address_space(3))) bf16x8_t;
    auto read_frags = [&](int step, bf16x8_t (&a)[FM], bf16x8_t (&b)[NB][3]) {
        const lds_char* cur = lds + (step % GS_NS) * S::BYTES;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) a[fm] = *(LdsFrag*)(cur + a_rd[fm]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int p = 0; p < 3; ++p) b[nb][p] = *(LdsFrag*)(cur + b_rd[nb] + p * TE * 64);
    };
    // the MFMAs of row blocks 2h, 2h + 1 (per 16-expert block: the plane of the smallest
    // parts first)
    auto mfma_half = [&](int h, const bf16x8_t (&a)[FM], const bf16x8_t (&b)[NB][3]) {
#pragma unroll
        for (int fm = 2 * h; fm < 2 * h + 2; ++fm)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                acc[fm][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], b[nb][2], acc[fm][nb], 0, 0, 0);
                acc[fm][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], b[nb][1], acc[fm][nb], 0, 0, 0);
                acc[fm][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], b[nb][0], acc[fm][nb], 0, 0, 0);
            }
    };
    // Step s: half of its MFMAs from fragments already in registers, then the barrier
    // (every wavefront's DMA of step s + 1 has landed and every read of stage s is done),
    // the DMA of step s + GS_NS into the stage s just freed, the fragment reads of step
    // s + 1 into the other register set, and the other half of the MFMAs, which cover
    // the barrier and the read latency.
    auto step = [&](int s, const bf16x8_t (&a)[FM], const bf16x8_t (&b)[NB][3], bf16x8_t (&an)[FM],
                    bf16x8_t (&bn)[NB][3]) {
        mfma_half(0, a, b);
        gs_sched_fence();
        wait_dma(std::integral_constant<int, GS_NS - 2>{});
        gs_step_barrier();
        dma(s + GS_NS);
        read_frags(s + 1, an, bn);
        gs_sched_fence();
        mfma_half(1, a, b);
        gs_sched_fence();
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) gs_pin_acc(acc[fm][nb]);
    };
    if (KT > 0) {
#pragma unroll
        for (int st = 0; st < GS_NS; ++st) dma(st);
        wait_dma(std::integral_constant<int, GS_NS - 1>{});
        gs_step_barrier();
        bf16x8_t a0[FM], b0[NB][3], a1[FM], b1[NB][3];
        read_frags(0, a0, b0);
        int s = 0;
        for (; s + 1 < KT; s += 2) {
            step(s, a0, b0, a1, b1);
            step(s + 1, a1, b1, a0, b0);
        }
        if (s < KT) step(s, a0, b0, a1, b1);
        wait_vmcnt<0>();                        // the zero loads past the K range land before exit
    }
    float* o = out + (size_t)blockIdx.z * T * E;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int e = e0 + wn * (TE / 2) + 16 * nb + fr;
        if (e >= E) continue;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = m0 + 64 * wm + fm * 16 + 4 * fq + v;
                if (t < T) o[(size_t)t * E + e] = acc[fm][nb][v];
            }
    }
}

// ------------------------------------------------------------------------- top-k
// Ranking key of a score: keys compare as the scores do under IEEE ordering, with
// -0 == +0 (both map to the key of +0); a NaN score gets key 0, below every number.
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (s != s) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of score_key on numbers (NaN keys decode to a NaN).
__device__ __forceinline__ float key_score(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Reductions over each row of 16 lanes, the result in every lane of the row: DPP steps
// that swap neighbours, swap pairs, mirror the half rows and mirror the rows.  Every
// lane combines the same values in the same pairs, so a sum is the same bits in all 16.
template <typename F>
__device__ __forceinline__ uint32_t row_reduce_u32(uint32_t v, F op) {
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));   // row_mirror
    return v;
}
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
    return row_reduce_u32(v, [](uint32_t a, uint32_t b) { return max(a, b); });
}
__device__ __forceinline__ float row_max_f32(float v) {
    return __uint_as_float(row_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
        return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
    }));
}
__device__ __forceinline__ float row_sum_f32(float v) {
    return __uint_as_float(row_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    }));
}

// Sixteen lanes per token, four tokens per wavefront, sixteen per workgroup; lane j of a
// token's row holds experts 4j .. 4j + 3, 64 + 4j .. 64 + 4j + 3, ... (up to 256).
// `logits` holds `nparts` partial sums [nparts][T][E] (split K); they are added in
// order and, when `logits_out` is given, the sum is written there.
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int nparts,
                                              float* __restrict__ logits_out,
                                              const float* __restrict__ bias,
                                              int32_t* __restrict__ topk_idx,
                                              float* __restrict__ topk_w,
                                              long long T, int E, int k, unsigned flags) {
    const int sub = threadIdx.x & 15;
    const long long t_row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
    const bool row_live = t_row < T;
    const long long t = row_live ? t_row : T - 1;   // a row past T repeats the last token, unstored
    const bool select_only = flags & MOE_FLAG_BIAS_SELECT_ONLY;
    const bool no_renorm = flags & MOE_FLAG_NO_RENORM;
    constexpr int NQ = 16;
    // expert of slot q: four runs of four consecutive experts, 64 apart, so that one
    // 16-byte load per lane reads 256 contiguous bytes of a token's row; within a lane
    // the slots run in expert order
    auto eid = [&](int q) { return 4 * sub + 64 * (q >> 2) + (q & 3); };
    const bool vec = (E & 3) == 0 && ((uintptr_t)logits & 15) == 0;
    auto load_part = [&](const float* row, float (&v)[NQ]) {
        if (vec) {
#pragma unroll
            for (int gq = 0; gq < NQ / 4; ++gq) {
                const int e0 = eid(4 * gq);
                const float4 f = e0 < E ? *reinterpret_cast<const float4*>(row + e0) : make_float4(0.f, 0.f, 0.f, 0.f);
                v[4 * gq] = f.x;
                v[4 * gq + 1] = f.y;
                v[4 * gq + 2] = f.z;
                v[4 * gq + 3] = f.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < NQ; ++q) v[q] = eid(q) < E ? row[eid(q)] : 0.f;
        }
    };
    float l[NQ];
    load_part(logits + t * E, l);
    // the later partial sums, added in part order
    for (int p = 1; p < nparts; ++p) {
        float v[NQ];
        load_part(logits + (long long)p * T * E + t * E, v);
#pragma unroll
        for (int q = 0; q < NQ; ++q) l[q] += v[q];
    }
    // ranking keys of the scores l + b (one fp32 add), plus one; 0 marks no candidate
    // (an expert past E, or one already chosen)
    uint32_t key1[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int e = eid(q);
        if (e < E && logits_out && row_live) logits_out[t * E + e] = l[q];
        const float b = (e < E && bias) ? bias[e] : 0.f;
        key1[q] = e < E ? score_key(l[q] + b) + 1u : 0u;   // keys stay below 0xFF800001
    }
    // Selection: each round takes the largest key of the row, and of equal keys the
    // lowest expert index (within a lane the first of equal keys is the lower index),
    // and retires it.
    int sel_i[8];
    uint32_t sel_k[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        sel_i[j] = 0;
        sel_k[j] = 0;
        if (j < k) {
            uint32_t bk = 0;
            int bq = 0;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const bool take = key1[q] > bk;
                bk = take ? key1[q] : bk;
                bq = take ? q : bq;
            }
            const uint32_t M = row_max_u32(bk);            // > 0: every row has k <= E experts
            const uint32_t mine = (bk != 0u && bk == M) ? (uint32_t)eid(bq) : 0xFFFFFFFFu;
            const uint32_t ew = ~row_max_u32(~mine);        // the lowest expert index at key M
            sel_i[j] = (int)ew;
            sel_k[j] = M - 1u;
            const int rq = mine == ew ? bq : -1;
#pragma unroll
            for (int q = 0; q < NQ; ++q) key1[q] = q == rq ? 0u : key1[q];
        }
    }
    // the values the gates come from: the ranking scores (decoded from the keys), or with
    // the selection-only bias the raw logits of the chosen experts
    float sel_g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        sel_g[j] = key_score(sel_k[j]);
        if (select_only && j < k) {
            const int e = sel_i[j];
            float own = 0.f;
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                if (eid(q) == e) own = l[q];
            // exactly one lane of the row holds expert e: the others contribute +0 bits
            sel_g[j] = __uint_as_float(row_max_u32(((e & 63) >> 2) == sub ? __float_as_uint(own) : 0u));
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
        float gv[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int e = eid(q);
            gv[q] = (select_only || !bias || e >= E) ? l[q] : l[q] + bias[e];
            if (e < E) gm = fmaxf(gm, gv[q]);
        }
        m = row_max_f32(gm);
        float part = 0.f;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            if (eid(q) < E) part += expf(gv[q] - m);
        den = row_sum_f32(part);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < k) den += expf(sel_g[j] - m);
    }
    if (row_live && sub < k) {
        float gj = 0.f;
        int ij = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j == sub) { gj = sel_g[j]; ij = sel_i[j]; }
        topk_idx[t * k + sub] = ij;
        topk_w[t * k + sub] = expf(gj - m) / den;
    }
}

// -------------------------------------------------------------------- launchers
// Tile of the gate projection: 16 tokens for short batches (fp32 MFMA), 64 for fp32 x,
// and 256 tokens x 64 or 128 experts for bf16 x (split weights, 512 threads).
int gate_tile_rows(long long T, int dtype) { return T <= 256 ? 16 : (dtype == MOE_F32 ? 64 : 256); }
int gate_tile_experts(long long T, int E, int dtype) {
    return (T > 256 && dtype != MOE_F32 && E > 64) ? 128 : GT_E;
}

// K ranges of the gate projection: enough workgroups for the CUs.  The bf16 tiles hold one
// workgroup per CU (160 KB of LDS), so they aim at 256 workgroups; the fp32 tiles at 512.
int gate_splits(long long T, int H, int E, int dtype) {
    if (T <= 0) return 1;
    const long long tm = gate_tile_rows(T, dtype), te = gate_tile_experts(T, E, dtype);
    const long long base = ((T + tm - 1) / tm) * ((E + te - 1) / te);
    const long long aim = tm == 256 ? 256 : 512;
    long long sp = (aim + base - 1) / base;
    const long long maxs = (H + 255) / 256;
    if (sp > maxs) sp = maxs;
    return (int)(sp < 1 ? 1 : sp);
}

bool gate_uses_planes(long long T, int dtype) { return T > 256 && dtype != MOE_F32; }

hipError_t launch_gate_logits(const void* x, int dtype, const float* wg, float* out, long long T, int H,
                              int E, int splits, bf16_t* planes, hipStream_t st) {
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
        const int te = gate_tile_experts(T, E, dtype);
        const dim3 grid((unsigned)((T + 255) / 256), (unsigned)((E + te - 1) / te), (unsigned)splits);
        const dim3 blk2(512);
        if (planes) {
            hipLaunchKernelGGL(k_gate_split_planes, dim3((unsigned)((H + 63) / 64), (unsigned)((E + 63) / 64)),
                               dim3(256), 0, st, wg, planes, H, E);
            if (te == 128)
                hipLaunchKernelGGL((k_gate_logits_p3<128>), grid, blk2, GateStage<128>::LDS, st, (const bf16_t*)x,
                                   planes, out, (int)T, H, E, kchunk);
            else
                hipLaunchKernelGGL((k_gate_logits_p3<64>), grid, blk2, GateStage<64>::LDS, st, (const bf16_t*)x,
                                   planes, out, (int)T, H, E, kchunk);
            return hipGetLastError();
        }
        if (te == 128)
            hipLaunchKernelGGL((k_gate_logits_x3<128>), grid, blk2, 0, st, (const bf16_t*)x, wg, out, (int)T, H, E, kchunk);
        else
            hipLaunchKernelGGL((k_gate_logits_x3<64>), grid, blk2, 0, st, (const bf16_t*)x, wg, out, (int)T, H, E, kchunk);
    }
    return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int nparts, float* logits_out, const float* bias, int32_t* idx,
                       float* w, long long T, int E, int k, unsigned flags, hipStream_t st) {
    hipLaunchKernelGGL(k_topk, dim3((unsigned)((T + 15) / 16)), dim3(256), 0, st,
                       logits, nparts, logits_out, bias, idx, w, T, E, k, flags);
    return hipGetLastError();
}

}  // namespace moe
