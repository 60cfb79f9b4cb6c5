// Grouped expert FFN: every expert's GEMMs in one launch per projection.
//
// Pages cited (by title and section):
//   [FourStage]  "MoE显存与计算开销四阶段手算指南" (bjdmk.com.cn/news/5154310)
//   [Principles] "MoE混合专家模型计算原理与推理部署实战解析" (sheratonhq.com/news/207562)
//
// [FourStage §4.3]: one kernel serves all active experts, driven by the per-expert row
// offsets of one contiguous input buffer, instead of one GEMM launch per expert.  Here
// the offsets become a device-side tile list (expert, first row, last row) and a
// persistent grid walks tile x column-block work items; the host never reads the
// per-expert counts.
//   first projection : h = act(rows @ W_in[e]) (* rows @ W_up[e] for SwiGLU)
//                      ([Principles §3.1] SwiGLU; [FourStage §2] SiLU FFN)
//   second projection: y = h @ W_out[e]
//
// bf16 kernel, for gfx950:
//   * v_mfma_f32_16x16x32_bf16, fp32 accumulation; workgroup = 4 wavefronts.
//   * K is staged through LDS 64 at a time, two stages, one barrier per step; the
//     next step's global loads are in flight while the current step's MFMAs run.
//   * Weights are [in, out] (N contiguous), but MFMA operands need 8 consecutive k per
//     lane.  Each thread loads an 8(k) x 8(n) block with eight 16-byte loads and
//     transposes it in registers with v_perm_b32 before a 16-byte LDS store, so both
//     operands sit k-contiguous in LDS.
//   * LDS rows are 64 bf16 = eight 16-byte chunks; chunk q of row n is stored at
//     q ^ swz(n), swz(n) = ((n >> 1) ^ (n >> 4)) & 7, which keeps both the fragment
//     reads (16 consecutive rows) and the transposed stores (rows 8 apart) free of
//     bank conflicts.
//   * Rows past the expert's end skip their MFMAs (per 16-row block), so short
//     experts cost little more than streaming their weights.
//   * Work items are ordered (super-group of `gm` row tiles) x column block x row tile,
//     and workgroup ids are remapped so that consecutive items run together on one XCD
//     (ids are dealt round-robin to the 8 XCDs): row tiles that share a weight slice,
//     and column blocks that share a row tile, meet in the same L2.
//   * The epilogue applies SiLU / SwiGLU in fp32, rounds to bf16 once, stages the tile
//     in LDS and writes whole rows with 16-byte stores.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int BK = 64;

__device__ __forceinline__ int swz(int n) { return ((n >> 1) ^ (n >> 4)) & 7; }

template <int BM, int BN, int NMAT, int WAVES_M>
struct GemmShape {
    static constexpr int WAVES_N = 4 / WAVES_M;
    static constexpr int BNm = BN / NMAT;          // columns per matrix = output columns
    static constexpr int WTM = BM / WAVES_M;       // wave tile rows
    static constexpr int WTN = BN / WAVES_N;       // wave tile LDS columns
    static constexpr int FM = WTM / 16;
    static constexpr int FN = WTN / 16;
    static constexpr int A_CHUNKS = BM * 8;        // 16-byte chunks of one A stage
    static constexpr int NA = (A_CHUNKS + 255) / 256;
    static constexpr int CS_STRIDE = BNm + 8;      // bf16 per row of the output staging tile
    static constexpr size_t STAGE_BYTES = (size_t)2 * (BM + BN) * BK * 2;
    static constexpr size_t OUT_BYTES = (size_t)BM * CS_STRIDE * 2;
    static constexpr size_t LDS_BYTES = STAGE_BYTES > OUT_BYTES ? STAGE_BYTES : OUT_BYTES;
};

template <int BM, int BN, int NMAT, int WAVES_M, int ACT, bool GATHER>
__global__ __launch_bounds__(256, 1) void k_grouped_gemm_bf16(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ gather_rows,
    const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1, bf16_t* __restrict__ C,
    const Tile* __restrict__ tiles, const int32_t* __restrict__ ntiles_p, int K, int N, int gm) {
    using S = GemmShape<BM, BN, NMAT, WAVES_M>;
    constexpr int WAVES_N = S::WAVES_N, BNm = S::BNm, WTM = S::WTM, FM = S::FM, FN = S::FN;
    constexpr int NA = S::NA, A_CHUNKS = S::A_CHUNKS;
    static_assert(NMAT * 8 * (BNm / 8) == 256, "one 8x8 weight block per thread");
    static_assert(NMAT == 1 || FN % 2 == 0, "SwiGLU waves hold gate and up halves");

    extern __shared__ uint4 smem[];
    uint4* sA = smem;                  // [2][BM][8]
    uint4* sB = smem + 2 * BM * 8;     // [2][BN][8]
    bf16_t* sC = reinterpret_cast<bf16_t*>(smem);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int l16 = lane & 15, lq = lane >> 4;

    const int NT = (N + BNm - 1) / BNm;
    const int KT = (K + BK - 1) / BK;
    const int ntiles = *ntiles_p;
    const long long total = (long long)ntiles * NT;
    const int G = gridDim.x;                          // multiple of 8
    const long long first = (long long)(blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

    // weight loader: thread -> (matrix, k block, column octet)
    constexpr int NBm = BNm / 8;
    const int nb = tid % NBm, kb = (tid / NBm) & 7, mat = tid / (NBm * 8);
    const uint32_t sel_even = (nb & 1) ? 0x07060302u : 0x05040100u;
    const uint32_t sel_odd = (nb & 1) ? 0x05040100u : 0x07060302u;
    int bdst[8];                                      // LDS chunk index (within a stage)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int n = mat * BNm + 8 * nb + (c ^ (nb & 1));
        bdst[c] = n * 8 + (kb ^ swz(n));
    }
    // row-operand loader: thread -> (row, 16-byte chunk)
    const int kc = tid & 7;
    int adst[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int r = (tid >> 3) + 32 * i;
        adst[i] = r * 8 + (kc ^ swz(r));
    }

    for (long long w = first; w < total; w += G) {
        // decode the work item
        const long long grp = w / ((long long)gm * NT);
        const long long rem = w - grp * gm * NT;
        const int gs = (int)min((long long)gm, (long long)ntiles - grp * gm);
        const int nt = (int)(rem / gs);
        const int mt = (int)(grp * gm + rem % gs);
        const Tile tl = tiles[mt];
        const int rows = tl.row1 - tl.row0;
        const int n0 = nt * BNm;

        const bf16_t* arow[NA];
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int r = min((tid >> 3) + 32 * i, rows - 1);
            long long g = tl.row0 + r;
            if constexpr (GATHER) g = gather_rows[g];
            arow[i] = A + g * (long long)K + kc * 8;
        }
        const bf16_t* bsrc = (mat ? B1 : B0) + (long long)tl.e * K * N + n0 + 8 * nb;
        const bool bcol = (n0 + 8 * nb) < N;
        const int vfm = max(0, min(FM, (rows - wm * WTM + 15) / 16));

        f32x4_t acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        uint4 ra[NA], rb[8];
        auto gload = [&](int kt) {
            const int k0 = kt * BK;
#pragma unroll
            for (int i = 0; i < NA; ++i) {
                ra[i] = uint4{0u, 0u, 0u, 0u};
                if ((A_CHUNKS % 256 == 0 || tid + 256 * i < A_CHUNKS) && k0 + kc * 8 < K)
                    ra[i] = *reinterpret_cast<const uint4*>(arow[i] + k0);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int kk = k0 + 8 * kb + i;
                rb[i] = uint4{0u, 0u, 0u, 0u};
                if (bcol && kk < K) rb[i] = *reinterpret_cast<const uint4*>(bsrc + (long long)kk * N);
            }
        };
        auto lstore = [&](int st) {
            uint4* a = sA + st * BM * 8;
#pragma unroll
            for (int i = 0; i < NA; ++i)
                if (A_CHUNKS % 256 == 0 || tid + 256 * i < A_CHUNKS) a[adst[i]] = ra[i];
            uint4* b = sB + st * BN * 8;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t sel = (c & 1) ? sel_odd : sel_even;
                const int d = c >> 1;
                auto dw = [&](const uint4& v) { return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w; };
                uint4 o;
                o.x = __builtin_amdgcn_perm(dw(rb[1]), dw(rb[0]), sel);
                o.y = __builtin_amdgcn_perm(dw(rb[3]), dw(rb[2]), sel);
                o.z = __builtin_amdgcn_perm(dw(rb[5]), dw(rb[4]), sel);
                o.w = __builtin_amdgcn_perm(dw(rb[7]), dw(rb[6]), sel);
                b[bdst[c]] = o;
            }
        };
        auto compute = [&](int st) {
            const uint4* a = sA + st * BM * 8;
            const uint4* b = sB + st * BN * 8;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int q = 4 * s + lq;
                bf16x8_t af[FM], bfr[FN];
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const int r = wm * WTM + 16 * fm + l16;
                    if (fm < vfm) af[fm] = __builtin_bit_cast(bf16x8_t, a[r * 8 + (q ^ swz(r))]);
                }
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    int n;
                    if constexpr (NMAT == 1)
                        n = wn * S::WTN + 16 * fn + l16;
                    else
                        n = (fn < FN / 2 ? 0 : BNm) + wn * (BNm / WAVES_N) + 16 * (fn % (FN / 2)) + l16;
                    bfr[fn] = __builtin_bit_cast(bf16x8_t, b[n * 8 + (q ^ swz(n))]);
                }
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    if (fm < vfm) {
#pragma unroll
                        for (int fn = 0; fn < FN; ++fn)
                            acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bfr[fn],
                                                                                 acc[fm][fn], 0, 0, 0);
                    }
                }
            }
        };

        gload(0);
        lstore(0);
        __syncthreads();
        for (int kt = 0; kt < KT; ++kt) {
            const int st = kt & 1;
            if (kt + 1 < KT) gload(kt + 1);
            compute(st);
            if (kt + 1 < KT) lstore(st ^ 1);
            __syncthreads();
        }

        // epilogue: activation, one rounding to bf16, staged through LDS
        constexpr int FO = (NMAT == 2) ? FN / 2 : FN;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            if (fm >= vfm) continue;
#pragma unroll
            for (int fo = 0; fo < FO; ++fo) {
                const int col = (NMAT == 2 ? wn * (BNm / WAVES_N) : wn * S::WTN) + 16 * fo + l16;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float val = acc[fm][fo][v];
                    if constexpr (NMAT == 2) val = silu_f32(val) * acc[fm][fo + FN / 2][v];
                    else if constexpr (ACT == 1) val = silu_f32(val);
                    const int r = wm * WTM + 16 * fm + 4 * lq + v;
                    sC[r * S::CS_STRIDE + col] = f32_to_bf16(val);
                }
            }
        }
        __syncthreads();
        constexpr int CPR = BNm / 8;     // 16-byte chunks per output row
        for (int c = tid; c < rows * CPR; c += 256) {
            const int r = c / CPR, cc = c % CPR;
            const int col = n0 + cc * 8;
            if (col < N)
                *reinterpret_cast<uint4*>(C + (long long)(tl.row0 + r) * N + col) =
                    *reinterpret_cast<const uint4*>(sC + r * S::CS_STRIDE + cc * 8);
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------------ tile list
// One workgroup of 256 threads (E <= 256): expert e gets ceil(count_e / BM) tiles.
__global__ __launch_bounds__(256) void k_build_tiles(const int32_t* __restrict__ offsets, int E,
                                                     int BM, Tile* __restrict__ tiles,
                                                     int32_t* __restrict__ ntiles) {
    __shared__ int buf[2][256];
    const int e = threadIdx.x;
    int r0 = 0, r1 = 0, nt = 0;
    if (e < E) {
        r0 = offsets[e];
        r1 = offsets[e + 1];
        nt = (r1 - r0 + BM - 1) / BM;
    }
    int cur = 0;
    buf[0][e] = nt;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const int v = buf[cur][e] + (e >= off ? buf[cur][e - off] : 0);
        buf[cur ^ 1][e] = v;
        cur ^= 1;
        __syncthreads();
    }
    const int incl = buf[cur][e];
    const int base = incl - nt;
    for (int i = 0; i < nt; ++i) tiles[base + i] = Tile{e, r0 + i * BM, min(r0 + (i + 1) * BM, r1), 0};
    if (e == 255) *ntiles = incl;
}

hipError_t launch_build_tiles(const int32_t* offsets, int E, int BM, Tile* tiles,
                              int32_t* ntiles, hipStream_t st) {
    hipLaunchKernelGGL(k_build_tiles, dim3(1), dim3(256), 0, st, offsets, E, BM, tiles, ntiles);
    return hipGetLastError();
}

int gemm_cfg_bm(GemmCfg c) {
    switch (c) {
        case GEMM_M16: return 16;
        case GEMM_M64: return 64;
        case GEMM_M128: return 128;
        default: return 256;
    }
}

// ------------------------------------------------------------------------ launching
template <int BM, int NMAT, int WAVES_M, int ACT, bool GATHER>
static hipError_t run_gemm(const void* A, const int32_t* gather_rows, const void* B0,
                           const void* B1, void* C, const Tile* tiles, const int32_t* ntiles,
                           long long max_items, int K, int N, int gm, hipStream_t st) {
    using S = GemmShape<BM, 256, NMAT, WAVES_M>;
    auto kern = k_grouped_gemm_bf16<BM, 256, NMAT, WAVES_M, ACT, GATHER>;
    static bool attr_set = false;   // per process; the attribute is a property of the code object
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)S::LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    int occ = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, 256, S::LDS_BYTES) != hipSuccess || occ < 1)
        occ = 1;
    long long G = (long long)device_cu_count() * occ;
    const long long cap = ((max_items + 7) / 8) * 8;
    if (G > cap) G = cap;
    G = ((G + 7) / 8) * 8;
    if (G < 8) G = 8;
    hipLaunchKernelGGL(kern, dim3((unsigned)G), dim3(256), S::LDS_BYTES, st,
                       (const bf16_t*)A, gather_rows, (const bf16_t*)B0, (const bf16_t*)B1,
                       (bf16_t*)C, tiles, ntiles, K, N, gm);
    return hipGetLastError();
}

template <int BM, int WAVES_M>
static hipError_t run_ffn(const void* a, const int32_t* gather_rows, const void* w_in,
                          const void* w_up, const void* w_out, void* h, void* y,
                          const Tile* tiles, const int32_t* ntiles, long long max_tiles,
                          int H, int F, int swiglu, int gm, hipStream_t st) {
    hipError_t e;
    const long long items1 = max_tiles * ((F + (swiglu ? 127 : 255)) / (swiglu ? 128 : 256));
    if (swiglu) {
        e = gather_rows ? run_gemm<BM, 2, WAVES_M, 1, true>(a, gather_rows, w_in, w_up, h, tiles, ntiles, items1, H, F, gm, st)
                        : run_gemm<BM, 2, WAVES_M, 1, false>(a, nullptr, w_in, w_up, h, tiles, ntiles, items1, H, F, gm, st);
    } else {
        e = gather_rows ? run_gemm<BM, 1, WAVES_M, 1, true>(a, gather_rows, w_in, nullptr, h, tiles, ntiles, items1, H, F, gm, st)
                        : run_gemm<BM, 1, WAVES_M, 1, false>(a, nullptr, w_in, nullptr, h, tiles, ntiles, items1, H, F, gm, st);
    }
    if (e != hipSuccess) return e;
    const long long items2 = max_tiles * ((H + 255) / 256);
    return run_gemm<BM, 1, WAVES_M, 0, false>(h, nullptr, w_out, nullptr, y, tiles, ntiles, items2, F, H, gm, st);
}

hipError_t launch_grouped_ffn_bf16(const void* a, const int32_t* gather_rows,
                                   const void* w_in, const void* w_up, const void* w_out,
                                   void* h, void* y, const Tile* tiles, const int32_t* ntiles,
                                   long long max_tiles, GemmCfg cfg, int H, int F, int swiglu,
                                   int gm, hipStream_t st) {
    switch (cfg) {
        case GEMM_M16:
            return run_ffn<16, 1>(a, gather_rows, w_in, w_up, w_out, h, y, tiles, ntiles, max_tiles, H, F, swiglu, gm, st);
        case GEMM_M64:
            return run_ffn<64, 1>(a, gather_rows, w_in, w_up, w_out, h, y, tiles, ntiles, max_tiles, H, F, swiglu, gm, st);
        case GEMM_M128:
            return run_ffn<128, 2>(a, gather_rows, w_in, w_up, w_out, h, y, tiles, ntiles, max_tiles, H, F, swiglu, gm, st);
        default:
            return run_ffn<256, 2>(a, gather_rows, w_in, w_up, w_out, h, y, tiles, ntiles, max_tiles, H, F, swiglu, gm, st);
    }
}

// ------------------------------------------------------------------- fp32 grouped FFN
// Plain LDS-tiled fp32 FMA kernel (64 rows x 64 output columns per workgroup, 4x4 per
// thread) for fp32 layers; one launch covers every (tile, column block).
template <int NMAT, int ACT, bool GATHER>
__global__ __launch_bounds__(256) void k_grouped_gemm_f32(
    const float* __restrict__ A, const int32_t* __restrict__ gather_rows,
    const float* __restrict__ B0, const float* __restrict__ B1, float* __restrict__ C,
    const Tile* __restrict__ tiles, const int32_t* __restrict__ ntiles_p, int K, int N) {
    constexpr int TM = 64, TN = 64, TK = 16;
    __shared__ float sA[TK][TM + 4];
    __shared__ float sB[NMAT][TK][TN + 4];
    const int ntl = *ntiles_p;
    const int mt = blockIdx.x, nt = blockIdx.y;
    if (mt >= ntl) return;
    const Tile tl = tiles[mt];
    const int rows = tl.row1 - tl.row0;
    const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
    const int n0 = nt * TN;
    float acc[NMAT][4][4] = {};
    // loader mappings
    const int ar = tid >> 2, aq = (tid & 3) * 4;
    long long ag = tl.row0 + min(ar, rows - 1);
    if constexpr (GATHER) ag = gather_rows[ag];
    const float* arow = A + ag * (long long)K;
    const int bk = tid >> 4, bq = (tid & 15) * 4;
    for (int k0 = 0; k0 < K; k0 += TK) {
        float4 av = make_float4(0.f, 0.f, 0.f, 0.f);
        if (k0 + aq < K) av = *reinterpret_cast<const float4*>(arow + k0 + aq);
        sA[aq + 0][ar] = av.x;
        sA[aq + 1][ar] = av.y;
        sA[aq + 2][ar] = av.z;
        sA[aq + 3][ar] = av.w;
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            const float* Bm = (m ? B1 : B0) + (long long)tl.e * K * N;
            float4 bv = make_float4(0.f, 0.f, 0.f, 0.f);
            if (k0 + bk < K && n0 + bq < N) bv = *reinterpret_cast<const float4*>(Bm + (long long)(k0 + bk) * N + n0 + bq);
            *reinterpret_cast<float4*>(&sB[m][bk][bq]) = bv;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk) {
            const float4 a4 = *reinterpret_cast<const float4*>(&sA[kk][tr * 4]);
            const float a[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const float4 b4 = *reinterpret_cast<const float4*>(&sB[m][kk][tc * 4]);
                const float b[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[m][i][j] = fmaf(a[i], b[j], acc[m][i][j]);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = tr * 4 + i;
        const int col = n0 + tc * 4;
        if (r >= rows || col >= N) continue;
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v = acc[0][i][j];
            if constexpr (NMAT == 2) v = silu_f32(v) * acc[NMAT - 1][i][j];
            else if constexpr (ACT == 1) v = silu_f32(v);
            o[j] = v;
        }
        *reinterpret_cast<float4*>(C + (long long)(tl.row0 + r) * N + col) = make_float4(o[0], o[1], o[2], o[3]);
    }
}

hipError_t launch_grouped_ffn_f32(const void* a, const int32_t* gather_rows,
                                  const void* w_in, const void* w_up, const void* w_out,
                                  void* h, void* y, const Tile* tiles, const int32_t* ntiles,
                                  long long max_tiles, int H, int F, int swiglu,
                                  hipStream_t st) {
    const dim3 blk(256);
    const dim3 g1((unsigned)max_tiles, (unsigned)((F + 63) / 64));
    const float* A = (const float*)a;
    if (swiglu) {
        if (gather_rows)
            hipLaunchKernelGGL((k_grouped_gemm_f32<2, 1, true>), g1, blk, 0, st, A, gather_rows, (const float*)w_in, (const float*)w_up, (float*)h, tiles, ntiles, H, F);
        else
            hipLaunchKernelGGL((k_grouped_gemm_f32<2, 1, false>), g1, blk, 0, st, A, nullptr, (const float*)w_in, (const float*)w_up, (float*)h, tiles, ntiles, H, F);
    } else {
        if (gather_rows)
            hipLaunchKernelGGL((k_grouped_gemm_f32<1, 1, true>), g1, blk, 0, st, A, gather_rows, (const float*)w_in, nullptr, (float*)h, tiles, ntiles, H, F);
        else
            hipLaunchKernelGGL((k_grouped_gemm_f32<1, 1, false>), g1, blk, 0, st, A, nullptr, (const float*)w_in, nullptr, (float*)h, tiles, ntiles, H, F);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 g2((unsigned)max_tiles, (unsigned)((H + 63) / 64));
    hipLaunchKernelGGL((k_grouped_gemm_f32<1, 0, false>), g2, blk, 0, st, (const float*)h, nullptr, (const float*)w_out, nullptr, (float*)y, tiles, ntiles, F, H);
    return hipGetLastError();
}

}  // namespace moe
