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
// Top-k is one wavefront per token: each lane holds up to four experts, k rounds of a wave-wide arg-max pick
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

// W_g [H, E] fp32 -> three bf16 planes [3][E][H] (expert-major, k contiguous) with
// w = p0 + p1 + p2 exactly (split3_bf16), once per call, so that the gate projection's
// workgroups copy 16-byte runs of k instead of splitting and transposing weights each.
// Tile: 64 k x 64 experts through LDS (loads coalesced along E, stores along k).
__global__ __launch_bounds__(256) void k_gate_split_planes(const float* __restrict__ wg, bf16_t* __restrict__ planes,
                                                           int H, int E) {
    __shared__ float tile[64][65];
    const int k0 = blockIdx.x * 64, e0 = blockIdx.y * 64, tid = threadIdx.x;
    for (int i = tid; i < 64 * 64; i += 256) {
        const int r = i >> 6, c = i & 63;
        const int k = k0 + r, e = e0 + c;
        tile[r][c] = (k < H && e < E) ? wg[(size_t)k * E + e] : 0.f;
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
        *reinterpret_cast<uint4*>(planes + ((size_t)0 * E + e) * H + k) = vh;
        *reinterpret_cast<uint4*>(planes + ((size_t)1 * E + e) * H + k) = vm;
        *reinterpret_cast<uint4*>(planes + ((size_t)2 * E + e) * H + k) = vl;
    }
}

// The gate projection from the pre-split planes, with its operands streamed into LDS by
// direct-to-LDS buffer loads (no register staging: a register stage covered one 64-K step
// of MFMAs against a load latency about twice as long).  Tile: 256 tokens x TE experts,
// eight wavefronts in a 4 x 2 grid (64 tokens x TE/2 experts each, two per SIMD), K steps
// of 32.  A stage holds x (256 rows of 64 bytes) and the three planes (3 TE rows of 64
// bytes), rows swizzled with swa4 for the fragment reads; GS_NS stages, the DMA GS_LEAD
// steps ahead, one barrier per step.  Every step issues the same DMA (steps past the K
// range load zeros into a stage nobody reads), so each wavefront waits with a constant
// count.  MFMA order per step and 16-expert block: the plane of the smallest parts first.
constexpr int GS_NS = 4, GS_LEAD = GS_NS - 1;

// keeps an accumulator in AGPRs (the MFMA then accumulates in place)
__device__ __forceinline__ void gs_pin_acc(f32x4_t& a) { asm volatile("" : "+a"(a)); }
// one 16-byte-per-lane direct-to-LDS load (1 KB per wavefront) at dst
__device__ __forceinline__ void gs_dma(__amdgpu_buffer_rsrc_t r, lds_char* dst, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, off, 0, 0, 0);
}
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
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(planes, (uint32_t)((size_t)3 * E * H * 2));
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
                if (e < E) off[i] = (uint32_t)((((size_t)pl * E + e) * H + kbeg + 8 * q) * 2);
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
                const uint32_t o = (off[i] != kOOB && step < KT && kq[i] + dk < (uint32_t)kend) ? off[i] + dk * 2 : kOOB;
                gs_dma(isx[i] ? rx : rp, st + j * 1024, o);
            }
        }
    };
    auto wait_step = [&]() {                    // this wavefront's DMA of the current step has landed
        if (NI % 8 == 0 || wave < NI % 8) wait_vmcnt<S::DPW_HI * (GS_LEAD - 1)>();
        else wait_vmcnt<S::DPW_LO * (GS_LEAD - 1)>();
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
    if (KT > 0) {
#pragma unroll
        for (int st = 0; st < GS_LEAD; ++st) dma(st);
        for (int s = 0; s < KT; ++s) {
            wait_step();
            gs_step_barrier();                                  // reads of step s - 1 done; step s landed
            dma(s + GS_LEAD);                                   // into the stage step s - 1 used
            const lds_char* cur = lds + (s % GS_NS) * S::BYTES;
            bf16x8_t a[FM], b[NB][3];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) a[fm] = *(const __attribute__((address_space(3))) bf16x8_t*)(cur + a_rd[fm]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int p = 0; p < 3; ++p)
                    b[nb][p] = *(const __attribute__((address_space(3))) bf16x8_t*)(cur + b_rd[nb] + p * TE * 64);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    // the small parts first
                    acc[fm][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], b[nb][2], acc[fm][nb], 0, 0, 0);
                    acc[fm][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], b[nb][1], acc[fm][nb], 0, 0, 0);
                    acc[fm][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], b[nb][0], acc[fm][nb], 0, 0, 0);
                }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) gs_pin_acc(acc[fm][nb]);
        }
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
    float s[4], g[4], l[4];
    bool live[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        live[q] = lane + 64 * q < E;
        l[q] = live[q] ? logits[t * E + lane + 64 * q] : 0.f;
    }
    // the later partial sums, added in part order; loaded four parts at a time so that
    // the loads are in flight together
    for (int p = 1; p < nparts; p += 4) {
        float v[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[q][i] = (live[q] && p + i < nparts) ? logits[(long long)(p + i) * T * E + t * E + lane + 64 * q] : 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (p + i < nparts) l[q] += v[q][i];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        if (live[q] && logits_out) logits_out[t * E + e] = l[q];
        const float b = (live[q] && bias) ? bias[e] : 0.f;
        s[q] = l[q] + b;                    // one fp32 add: the ranking score
        g[q] = select_only ? l[q] : s[q];   // what the gate is computed from
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
// Tile of the gate projection: 16 tokens for short batches (fp32 MFMA), 64 for fp32 x,
// and 256 tokens x 64 or 128 experts for bf16 x (split weights, 512 threads).
int gate_tile_rows(long long T, int dtype) { return T <= 256 ? 16 : (dtype == MOE_F32 ? 64 : 256); }
int gate_tile_experts(long long T, int E, int dtype) {
    return (T > 256 && dtype != MOE_F32 && E > 64) ? 128 : GT_E;
}

// K ranges of the gate projection: enough workgroups for the CUs.  The bf16 tiles hold one
// workgroup per CU (92 KB of LDS), so they aim at 256 workgroups; the fp32 tiles at 512.
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
    hipLaunchKernelGGL(k_topk, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st,
                       logits, nparts, logits_out, bias, idx, w, T, E, k, flags);
    return hipGetLastError();
}

}  // namespace moe
