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
//   * Work items are ordered expert x column block x the expert's row tiles, and
//     workgroup ids are remapped so that consecutive items run together on one XCD
//     (ids are dealt round-robin to the 8 XCDs): row tiles that share a weight slice,
//     and column blocks that share a row tile, meet in the same L2.
//   * The epilogue applies SiLU / SwiGLU in fp32, rounds to bf16 once, stages the tile
//     in LDS and writes whole rows with 16-byte stores.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

// Work item w of a persistent grouped-GEMM launch -> (row tile mt, column block nt).
// Items are expert-major.  Within an expert, its row tiles are taken in groups of
// kItemRows and each group is walked column block by column block, so the items that
// run at the same time (consecutive ones, on one XCD) cover a few row tiles x several
// column blocks: each row tile's A operand is shared by several concurrent items and
// each weight slice by the group's row tiles, instead of every A tile being re-read
// for every column block when an expert has many row tiles.  An expert with at most
// kItemRows row tiles is walked column block by column block over all of them.
constexpr int kItemRows = 4;

__device__ __forceinline__ void item_coords(long long w, int NT, const Tile* __restrict__ tiles, int& mt,
                                            int& nt) {
    const Tile te = tiles[w / NT];
    const long long local = w - (long long)te.first * NT;           // < cnt * NT
    const int rg = (int)(local / ((long long)kItemRows * NT));      // row-tile group
    const int rows_in = min(kItemRows, te.cnt - rg * kItemRows);    // row tiles in this group
    const int j = (int)(local - (long long)rg * kItemRows * NT);
    nt = j / rows_in;
    mt = te.first + rg * kItemRows + j % rows_in;
}

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
    const Tile* __restrict__ tiles, const int32_t* __restrict__ ntiles_p, int K, int N) {
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
        // decode the work item (order: item_coords)
        int mt, nt;
        item_coords(w, NT, tiles, mt, nt);
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
        // Weight loads carry the non-temporal hint: this kernel serves decode-sized layers, where
        // each weight byte is read by one work item once (8% faster than plain loads on 64 tokens
        // of 64 SwiGLU experts).
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
                if (bcol && kk < K) rb[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(bsrc + (long long)kk * N)));
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

// --------------------------------------------- direct-to-LDS grouped GEMM (main path)
// The grouped GEMM for row tiles of 64..256 rows.  Both operands travel from HBM
// straight into LDS with buffer_load_dwordx4 ... lds (lane i's 16 bytes land in slot i
// of the wavefront's 1 KB); a buffer resource bounds each operand, so chunks past K,
// N or the tile's rows read as zeros and no register stages the tiles.
//   * A (rows, k-contiguous): LDS [BM][32], chunk q of row m at q ^ ((m >> 1) & 2);
//     fragments are ds_read_b128.
//   * W (k rows, n-contiguous), kept as in memory: LDS [32][256] (SiLU2 and the second
//     projection) or [2][32][128] (SwiGLU gate | up; 192 and 2 x 96 of them used by the
//     320-row tile), 16-byte chunk c of row k at
//     c ^ fk(k), fk(k) = 2 * ((k & 3) | ((k >> 3) & 1) << 2).  The MFMA operand (8
//     consecutive k of one column per lane) comes from two ds_read_b64_tr_b16 (gfx950):
//     within each group of 16 lanes, source lane j reads 4 consecutive columns of row
//     k0 + j/4 and lane i receives column i of those four rows.  Both swizzles keep
//     the lanes of one LDS cycle on distinct banks.
//   * Four LDS stages of 32 k with the DMA three steps ahead.  One K step runs in a
//     helper that takes the stage it reads and the stage it fills as separate
//     __restrict__ pointers, so the compiler knows the fragment reads do not touch the
//     buffer in flight and does not wait for it; the step's own wait is explicit
//     (s_waitcnt vmcnt(<DMA issued after this stage>)).
//   * 256 x 256 tile, 4 wavefronts of 128 x 128 (v_mfma_f32_16x16x32_bf16, fp32
//     accumulators in AGPRs), which halves the bytes moved per FLOP against 128-row
//     tiles; 128- and 64-row tiles use the same code with shorter wavefront tiles, and
//     the 320 x 192 tile with wavefront tiles of 160 x 96.
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));

// Zeroes one accumulator as a value of its own: with a zero constant shared by several
// accumulators, the register allocator may not update them in place in the K loop and
// then moves accumulators at every step.
__device__ __forceinline__ void acc_zero(f32x4_t& a) {
    a = f32x4_t{0.f, 0.f, 0.f, 0.f};
    asm volatile("" : "+a"(a));
}

__device__ __forceinline__ int fk(int k) { return 2 * ((k & 3) | (((k >> 3) & 1) << 2)); }
// 320-row tiles keep W rows of 384 bytes (SiLU2) or 192 bytes per matrix (SwiGLU): the
// 32-byte block b of row k sits at b ^ fk320(k), within groups of 4 (384-byte rows) or
// pairs (192-byte rows).  The rows one ds_read_b64_tr_b16 serves per LDS cycle (k0..k0+3
// and k0+8..k0+11) then land on 8 distinct 32-byte bank slots (row starts are 128 or 64
// bytes apart modulo 256).
template <int NMAT>
__device__ __forceinline__ int fk320(int k) {
    return NMAT == 1 ? (((k >> 1) & 1) | (((k >> 3) & 1) << 1)) : ((k >> 3) & 1);
}
// the LDS 32-byte block of logical W column block blk for a lane whose rows have swizzle g
template <int BM, int NMAT>
__device__ __forceinline__ int wblk(int blk, int g) {
    if constexpr (BM == 320) return NMAT == 1 ? ((blk & ~3) | ((blk & 3) ^ g)) : ((blk & ~1) | ((blk & 1) ^ g));
    else return (blk & ~7) | ((blk & 7) ^ g);
}
// A rows use the 64-byte row swizzle swa4 (common.h).
constexpr int kWStream = 2;                     // the nt bit of a buffer load's cache policy

// Tile shapes: BM x BN outputs (BN over both matrices for SwiGLU).  The 320-row tile is
// 192 wide so that its accumulators (60 16x16 blocks per wavefront) still fit the AGPRs;
// it lets one tile hold every row of an expert with up to 320 rows, so the expert's
// weight slice is streamed once.  The LDS weight rows stay LBN = 256 columns wide in
// every shape (only BN are filled and read), which keeps one swizzle for all of them.
template <int BM, int NMAT>
struct LdsShape {
    static constexpr int BN = BM == 320 ? 192 : 256, BNm = BN / NMAT, WAVES_M = 2, WAVES_N = 2, BK = 32;
    // A and W stages sit in rings of their own, NA and NW stages deep: the DMA of a step's
    // A runs NA - 1 steps ahead of its use, its W NW - 1 steps.  320-row tiles stream each
    // expert's weights from HBM once; their W runs 7 steps ahead (8 x 12 KB) against 2 for
    // A, which comes from L2 (3 x 20 KB), to keep enough weight bytes in flight for HBM's
    // latency.  They keep W rows 192 wide in LDS (the columns they use).
    static constexpr int NA = BM == 320 ? 3 : 4, NW = BM == 320 ? 8 : 4;
    static constexpr int LBN = BM == 320 ? 192 : 256, LBNm = LBN / NMAT;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N, FM = WTM / 16, FN = WTN / 16;
    static constexpr int A_STAGE = BM * BK * 2, B_STAGE = BK * LBN * 2;
    static constexpr int W_RING = NA * A_STAGE;       // LDS offset of the W ring
    static constexpr int ADMA = A_STAGE / 1024 / 4;   // A DMA instructions per wavefront per step
    static constexpr int BDMA = B_STAGE / 1024 / 4;   // W DMA instructions per wavefront per step
    static constexpr int DPW = ADMA + BDMA;
    static constexpr int BROW = 2 * LBNm;             // LDS bytes per W row
    static constexpr int BMAT_DMA = B_STAGE / 1024 / NMAT;   // W DMA instructions per matrix
    // Cache policy of the W loads.  The tile builder picks 320-row tiles when they hold an
    // expert's rows in fewer tiles, typically one, so each weight slice is read by one work
    // item: its loads carry the non-temporal hint (nt), and the streamed weights leave L2
    // before the A tiles the XCD's other items still re-read.  The pages' worked shape
    // measured 2.54 -> 2.41 ms on the first projection.  Where several row tiles share a
    // slice (the smaller tiles), the hint measured 15-18% slower, as it evicts the slice
    // between them.
    static constexpr int W_AUX = BM == 320 ? 2 : 0;
    static constexpr int CS_STRIDE = BNm + 8;
    static constexpr size_t RING_BYTES = (size_t)NA * A_STAGE + (size_t)NW * B_STAGE;
    static constexpr size_t LDS_BYTES = RING_BYTES > (size_t)BM * CS_STRIDE * 2 ? RING_BYTES
                                                                                : (size_t)BM * CS_STRIDE * 2;
    // Each step issues its A DMA (for step + NA - 1), then its W DMA (for step + NW - 1).
    // Before step r, A(r) and W(r) must have landed; loads complete in issue order, so the
    // wait is for the later-issued of the two: A(r) (issued NA - 1 steps back, followed by
    // its own step's W and NA - 2 more steps) when NW > NA, else W(r).
    static constexpr int VMCNT = NW > NA ? BDMA + (NA - 2) * DPW : (NW - 2) * DPW;
    static_assert(NW >= NA && NA >= 2, "the W ring is at least as deep as the A ring");
    static_assert((NW - 1) * DPW < 64, "DMA in flight fits the 6-bit vmcnt");
};


// Per-tile DMA description (one wavefront's share of a K step).
template <int ADMA, int BDMA>
struct DmaPlan {                 // (the buffer resources travel as separate arguments)
    uint32_t a_off[ADMA];        // byte offset of the lane's chunk at k0 = 0 (kOOB: none)
    uint32_t a_k[ADMA];          // first k of the lane's chunk
    uint32_t b_off[BDMA];        // byte offset at k0 = 0 (kOOB: column past N)
};

// This wavefront's share of the A DMA of K step kt into the A stage `dst`; `dummy` loads
// zeros (the prologue's placeholders, which keep every step's DMA count the same).
template <int BM, int NMAT>
__device__ __forceinline__ void dma_a(lds_char* dst, __amdgpu_buffer_rsrc_t ra,
                                      const DmaPlan<LdsShape<BM, NMAT>::ADMA, LdsShape<BM, NMAT>::BDMA>& pl,
                                      int kt, int K, int wave, bool dummy = false) {
    using S = LdsShape<BM, NMAT>;
    constexpr int ADMA = S::ADMA;
    const uint32_t k0 = (uint32_t)kt * S::BK;
#pragma unroll
    for (int i = 0; i < ADMA; ++i) {
        const uint32_t off = (!dummy && k0 + pl.a_k[i] < (uint32_t)K) ? pl.a_off[i] + k0 * 2 : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(dst + (wave * ADMA + i) * 1024), 16, off, 0, 0, 0);
    }
}

// This wavefront's share of the W DMA of K step kt into the W stage `dst`.
template <int BM, int NMAT>
__device__ __forceinline__ void dma_w(lds_char* dst, __amdgpu_buffer_rsrc_t rb0, __amdgpu_buffer_rsrc_t rb1,
                                      const DmaPlan<LdsShape<BM, NMAT>::ADMA, LdsShape<BM, NMAT>::BDMA>& pl,
                                      int kt, uint32_t rowB, int wave) {
    using S = LdsShape<BM, NMAT>;
    constexpr int BDMA = S::BDMA;
    const uint32_t k0 = (uint32_t)kt * S::BK;
#pragma unroll
    for (int i = 0; i < BDMA; ++i) {
        const int j = wave * BDMA + i;
        // rows k0 >= K fall past the resource's K * rowB bytes and read zeros (the host
        // keeps (K + 128) * rowB below 2^32, so the offset cannot wrap)
        const uint32_t off = pl.b_off[i] == kOOB ? kOOB : pl.b_off[i] + k0 * rowB;
        constexpr int per_mat = S::BMAT_DMA;   // instructions of the first matrix
        const __amdgpu_buffer_rsrc_t rb = (NMAT == 2 && j >= per_mat) ? rb1 : rb0;
        constexpr int aux = S::W_AUX;          // (a local: the host pass rejects the member here)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(dst + j * 1024), 16, off, 0, 0, aux);
    }
}

// One step's DMA: A of step r + NA - 1 and W of step r + NW - 1 (r relative to the first
// step kt0 of the work, absolute step kt0 + r), each into the stage its ring holds for it
// (the stage of step r - 1, free once every wavefront has passed step r's barrier).
template <int BM, int NMAT>
__device__ __forceinline__ void dma_step(lds_char* lds, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb0,
                                         __amdgpu_buffer_rsrc_t rb1,
                                         const DmaPlan<LdsShape<BM, NMAT>::ADMA, LdsShape<BM, NMAT>::BDMA>& pl,
                                         int kt0, int r, int K, uint32_t rowB, int wave) {
    using S = LdsShape<BM, NMAT>;
    const int ra_step = r + S::NA - 1, rw_step = r + S::NW - 1;
    dma_a<BM, NMAT>(lds + (ra_step % S::NA) * S::A_STAGE, ra, pl, kt0 + ra_step, K, wave);
    dma_w<BM, NMAT>(lds + S::W_RING + (rw_step % S::NW) * S::B_STAGE, rb0, rb1, pl, kt0 + rw_step, rowB, wave);
}

// Instruction I of one step's DMA (I < ADMA: A instruction I, else W instruction
// I - ADMA), with the targets of dma_step; lets the 320-row K step spread its DMA
// issues between its MFMAs.
template <int BM, int NMAT, int I>
__device__ __forceinline__ void dma_one(lds_char* lds, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb0,
                                        __amdgpu_buffer_rsrc_t rb1,
                                        const DmaPlan<LdsShape<BM, NMAT>::ADMA, LdsShape<BM, NMAT>::BDMA>& pl,
                                        int kt0, int r, int K, uint32_t rowB, int wave) {
    using S = LdsShape<BM, NMAT>;
    if constexpr (I < S::ADMA) {
        const int step = r + S::NA - 1;
        const uint32_t k0 = (uint32_t)(kt0 + step) * S::BK;
        lds_char* dst = lds + (step % S::NA) * S::A_STAGE + (wave * S::ADMA + I) * 1024;
        const uint32_t off = (k0 + pl.a_k[I] < (uint32_t)K) ? pl.a_off[I] + k0 * 2 : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)dst, 16, off, 0, 0, 0);
    } else {
        constexpr int i = I - S::ADMA;
        const int step = r + S::NW - 1;
        const uint32_t k0 = (uint32_t)(kt0 + step) * S::BK;
        const int j = wave * S::BDMA + i;
        lds_char* dst = lds + S::W_RING + (step % S::NW) * S::B_STAGE + j * 1024;
        const uint32_t off = pl.b_off[i] == kOOB ? kOOB : pl.b_off[i] + k0 * rowB;
        constexpr int per_mat = S::BMAT_DMA;
        const __amdgpu_buffer_rsrc_t rb = (NMAT == 2 && j >= per_mat) ? rb1 : rb0;
        constexpr int aux = S::W_AUX;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)dst, 16, off, 0, 0, aux);
    }
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// The DMA ahead of a work's first step, issued as the steps -(NW - 1) .. -1 would have
// issued it, so that the first steps wait with the same count as the rest: A of steps
// below 0 is a zero-loading placeholder.
template <int BM, int NMAT>
__device__ __forceinline__ void dma_prologue(lds_char* lds, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb0,
                                             __amdgpu_buffer_rsrc_t rb1,
                                             const DmaPlan<LdsShape<BM, NMAT>::ADMA, LdsShape<BM, NMAT>::BDMA>& pl,
                                             int kt0, int K, uint32_t rowB, int wave) {
    using S = LdsShape<BM, NMAT>;
#pragma unroll
    for (int r = -(S::NW - 1); r < 0; ++r) {
        const int ra_step = r + S::NA - 1, rw_step = r + S::NW - 1;
        const int aslot = ((ra_step % S::NA) + S::NA) % S::NA;
        dma_a<BM, NMAT>(lds + aslot * S::A_STAGE, ra, pl, kt0 + ra_step, K, wave, ra_step < 0);
        dma_w<BM, NMAT>(lds + S::W_RING + rw_step * S::B_STAGE, rb0, rb1, pl, kt0 + rw_step, rowB, wave);
    }
}

// One K step: read this step's fragments from `cur`, start the DMA of step kt_dma into
// `nxt`, and run the step's MFMAs with the DMA instructions spread between them (a
// burst of DMA issues at the start of the step can stall the wavefront while the
// texture-address queue drains).  Steps past the end of K load from an out-of-range
// offset, which reads zeros into a stage nobody reads, so every step issues the same
// number of DMA instructions and the wait count stays constant.  `cur` and `nxt` are
// distinct stages; saying so with __restrict__ lets the compiler issue the reads
// without waiting for DMA in flight.  Only the first FMA 16-row blocks of the wavefront
// tile hold rows of the tile (FMA < FM for short experts), so only they are read and
// multiplied.
template <int BM, int NMAT, int FMA>
__device__ __attribute__((always_inline)) inline void kstep(
    const lds_char* __restrict__ As, const lds_char* __restrict__ Bs, lds_char* __restrict__ lds,
    __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb0, __amdgpu_buffer_rsrc_t rb1,
    const DmaPlan<LdsShape<BM, NMAT>::ADMA, LdsShape<BM, NMAT>::BDMA>& pl, int kt0, int r, int K, uint32_t rowB,
    int wave, int a_rd, int b_rd, int g, int wn,
    f32x4_t (&acc)[FMA][LdsShape<BM, NMAT>::FN]) {
    using S = LdsShape<BM, NMAT>;
    constexpr int FM = FMA, FN = S::FN, BROW = S::BROW;
    // Every fragment read of the step is issued before its first MFMA (A row block 0,
    // then the B columns, then the other A row blocks, in the order the MFMAs use them),
    // so the MFMAs wait on the LDS counter step by step instead of paying the LDS
    // latency once per A row block.
    bf16x8_t af[FM], bfr[FN];
    auto read_a = [&](int fm) {
        af[fm] = *(const __attribute__((address_space(3))) bf16x8_t*)(As + a_rd + fm * 16 * S::BK * 2);
    };
    read_a(0);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        int mat, blk;                          // W matrix and its 16-column block
        if constexpr (NMAT == 1) {
            mat = 0;
            blk = wn * (S::WTN / 16) + fn;
        } else {
            mat = fn < FN / 2 ? 0 : 1;
            blk = wn * (FN / 2) + (fn % (FN / 2));
        }
        const lds_char* p = Bs + mat * S::BK * BROW + b_rd + (wblk<BM, NMAT>(blk, g) << 5);
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)p);
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(p + 4 * BROW));
        const v8i16_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        bfr[fn] = __builtin_bit_cast(bf16x8_t, v);
    }
#pragma unroll
    for (int fm = 1; fm < FM; ++fm) read_a(fm);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (BM == 320) {
        // one DMA instruction after each 16-row block's MFMAs (the rest after the last), in
        // an order the scheduler keeps: a burst of DMA issues could stall the wavefront on
        // the texture-address queue while the MFMA pipe has nothing queued
        constexpr int D = S::DPW;
        static_for<0, FM>([&](auto fmc) {
            constexpr int fm = decltype(fmc)::value;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
            if constexpr (fm < D) dma_one<BM, NMAT, fm>(lds, ra, rb0, rb1, pl, kt0, r, K, rowB, wave);
            __builtin_amdgcn_sched_barrier(0);
        });
        static_for<FM, D>([&](auto ic) {
            dma_one<BM, NMAT, decltype(ic)::value>(lds, ra, rb0, rb1, pl, kt0, r, K, rowB, wave);
        });
        return;
    }
    dma_step<BM, NMAT>(lds, ra, rb0, rb1, pl, kt0, r, K, rowB, wave);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
    // issue order: one DMA instruction, then FM*FN/DPW MFMAs, DPW times (the 320-row tile
    // interleaves by hand above: this pattern made the allocator move its accumulators)
    if constexpr (BM != 320) {
        constexpr int PER = FM * FN / S::DPW > 0 ? FM * FN / S::DPW : 1;
#pragma unroll
        for (int i = 0; i < S::DPW; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // VMEM read (the LDS DMA)
            __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);   // MFMA
        }
    }
}

template <int DPW>
__device__ __forceinline__ void wait_dma(int pending);
__device__ __forceinline__ void kloop_barrier();

// The K loop of one work item for a wavefront whose rows fill FMA 16-row blocks: KT
// steps starting at step kt0 (dma_prologue has issued the DMA ahead of the first).
template <int BM, int NMAT, int FMA>
__device__ __attribute__((always_inline)) inline void kloop(
    lds_char* lds, int KT, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb0, __amdgpu_buffer_rsrc_t rb1,
    const DmaPlan<LdsShape<BM, NMAT>::ADMA, LdsShape<BM, NMAT>::BDMA>& pl, int K, uint32_t rowB, int wave,
    int a_rd, int b_rd, int g, int wn, f32x4_t (&acc)[FMA][LdsShape<BM, NMAT>::FN], int kt0) {
    using S = LdsShape<BM, NMAT>;
    for (int r = 0; r < KT; ++r) {
        wait_vmcnt<S::VMCNT>();
        kloop_barrier();
        kstep<BM, NMAT, FMA>(lds + (r % S::NA) * S::A_STAGE, lds + S::W_RING + (r % S::NW) * S::B_STAGE, lds,
                             ra, rb0, rb1, pl, kt0, r, K, rowB, wave, a_rd, b_rd, g, wn, acc);
    }
}

// The 320-row K loop with the barrier of step r + 1 moved before the last 16-row block
// of step r: every wavefront has then read all of step r's fragments (lgkmcnt(0)) and
// issued step r's DMA, so the barrier means what it meant at the top of step r + 1.
// Step r + 1's first A block and B fragments are read right after it, while step r's
// last block of MFMAs runs, so the next step's MFMAs do not start behind a barrier
// and an LDS round trip.  Barriers per item: KT + 1 (one more than kloop; the DMA-only
// wavefronts of a 320-row tile add it after their loop).
template <int BM, int NMAT, int FMA>
__device__ __attribute__((always_inline)) inline void kloop_early(
    lds_char* lds, int KT, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb0, __amdgpu_buffer_rsrc_t rb1,
    const DmaPlan<LdsShape<BM, NMAT>::ADMA, LdsShape<BM, NMAT>::BDMA>& pl, int K, uint32_t rowB, int wave,
    int a_rd, int b_rd, int g, int wn, f32x4_t (&acc)[FMA][LdsShape<BM, NMAT>::FN], int kt0) {
    using S = LdsShape<BM, NMAT>;
    constexpr int FM = FMA, FN = S::FN, BROW = S::BROW, D = S::DPW;
    auto a_stage = [&](int r) -> const lds_char* { return lds + (r % S::NA) * S::A_STAGE; };
    auto b_stage = [&](int r) -> const lds_char* { return lds + S::W_RING + (r % S::NW) * S::B_STAGE; };
    auto read_a = [&](const lds_char* As, int fm) -> bf16x8_t {
        return *(const __attribute__((address_space(3))) bf16x8_t*)(As + a_rd + fm * 16 * S::BK * 2);
    };
    auto read_b = [&](const lds_char* Bs, int fn) -> bf16x8_t {
        int mat, blk;
        if constexpr (NMAT == 1) {
            mat = 0;
            blk = wn * (S::WTN / 16) + fn;
        } else {
            mat = fn < FN / 2 ? 0 : 1;
            blk = wn * (FN / 2) + (fn % (FN / 2));
        }
        const lds_char* p = Bs + mat * S::BK * BROW + b_rd + (wblk<BM, NMAT>(blk, g) << 5);
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)p);
        const v4i16_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(p + 4 * BROW));
        const v8i16_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8_t, v);
    };
    // a0 and bf: step r's first A block and B fragments, read while step r - 1 finished
    bf16x8_t a0, bf[FN];
    wait_vmcnt<S::VMCNT>();
    kloop_barrier();
    a0 = read_a(a_stage(0), 0);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) bf[fn] = read_b(b_stage(0), fn);
    for (int r = 0; r < KT; ++r) {
        bf16x8_t af[FM];
        af[0] = a0;
#pragma unroll
        for (int fm = 1; fm < FM; ++fm) af[fm] = read_a(a_stage(r), fm);
        __builtin_amdgcn_sched_barrier(0);
        // blocks 0 .. FM - 2, one DMA instruction after each block's first MFMA
        static_for<0, FM - 1>([&](auto fmc) {
            constexpr int fm = decltype(fmc)::value;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bf[fn], acc[fm][fn], 0, 0, 0);
            if constexpr (fm < D) dma_one<BM, NMAT, fm>(lds, ra, rb0, rb1, pl, kt0, r, K, rowB, wave);
            __builtin_amdgcn_sched_barrier(0);
        });
        static_for<FM - 1, D>([&](auto ic) {
            dma_one<BM, NMAT, decltype(ic)::value>(lds, ra, rb0, rb1, pl, kt0, r, K, rowB, wave);
        });
        // the barrier of step r + 1, also after the last step (the reads then take stages
        // nobody uses: no branch here, which would make the compiler copy the accumulators)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wait_vmcnt<S::VMCNT>();
        kloop_barrier();
        a0 = read_a(a_stage(r + 1), 0);
        // the last block: each B fragment is re-read for step r + 1 once its MFMA has taken it
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            acc[FM - 1][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[FM - 1], bf[fn], acc[FM - 1][fn], 0, 0, 0);
            bf[fn] = read_b(b_stage(r + 1), fn);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Workgroup barrier of the K loop.  Each wavefront has already waited for its own DMA
// of the step (wait_vmcnt) and its fragment reads of the previous step were consumed by
// MFMAs before it arrives, so the barrier alone makes the stage complete for all and the
// stage being refilled free.  It is written without __syncthreads' memory fence, which
// otherwise leads the compiler to drain every DMA in flight (vmcnt(0)) at each step; the
// memory clobber still keeps the compiler from moving memory operations across it.
__device__ __forceinline__ void kloop_barrier() { asm volatile("s_barrier" ::: "memory"); }
// s_waitcnt lgkmcnt(0) as the builtin (gfx9 encoding: vmcnt and expcnt at their maxima), so
// that the compiler knows the fragment reads have landed: after the same wait written as
// inline asm it put a redundant lgkmcnt wait before each MFMA of the next phase.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Split of the last round's items along K.  A persistent launch of G workgroups runs its
// items in rounds of G; when the last round is partial, its items are split along K into
// `split` parts, so that round is filled with shorter work.  Each part writes its fp32
// accumulators (in register layout) to a slot of the part buffer; the last part of an item
// to finish (counted with one atomic per item) adds all parts in part order, so the sum
// does not depend on which part finished last, and writes the output as an unsplit item
// would.  Nothing waits for another workgroup.
constexpr int kPartSlots = kGemmPartSlots;   // parts in flight at most (slots of the part buffer)
constexpr int kMaxSplit = 8;
constexpr int kMinPartSteps = 64;     // K steps per part at least (2048 of K)

struct SplitPart {
    float* buf;       // this part's slot; NULL when the item is not split
    float* item;      // the item's first slot (its `split` slots are consecutive)
    int* cnt;         // the item's arrival counter
    int split;
    size_t slot_floats;
};

// Decides the split of a launch and maps work index w to (item, part).
struct WorkSplit {
    long long full, nwork;
    int rem, split;
    __device__ WorkSplit(long long total, int G, int KT) {
        full = total / G * G;
        rem = (int)(total - full);
        split = 1;
        if (rem > 0 && KT >= 2 * kMinPartSteps) {
            const int by_slots = (G < kPartSlots ? G : kPartSlots) / rem;
            const int by_steps = KT / kMinPartSteps;
            split = min(min(by_slots, by_steps), kMaxSplit);
            if (split < 1) split = 1;
        }
        nwork = full + (long long)rem * split;
    }
    __device__ void item_of(long long w, long long& item, int& part, int& slot) const {
        if (split == 1 || w < full) {
            item = w;
            part = 0;
            slot = -1;
        } else {
            const int p = (int)(w - full);
            slot = p % rem;
            part = p / rem;
            item = full + slot;
        }
    }
};

// Parts travel through device-scope (sc1) buffer stores and loads: such accesses are
// coherent across the XCDs' L2 caches on their own, so the hand-off needs no L2-wide
// write-back or invalidate (which would also evict the tiles other workgroups on the
// XCD are reusing), only that this workgroup's part stores have completed before its
// arrival is counted.
constexpr int kDeviceScope = 16;      // the sc1 bit of a buffer access's cache policy

__device__ __forceinline__ void store_part(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f32x4_t v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, byte_off, 0, kDeviceScope);
}

__device__ __forceinline__ f32x4_t load_part(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kDeviceScope));
}

// Arrival of a workgroup that has written its part: returns (uniformly) whether it is the
// item's last part.  Every wavefront waits for its part stores to complete before the
// barrier that precedes the count, so when the count reaches `split` all parts are in
// place for the last arriver's device-scope loads.  `flag` is an LDS word outside the
// staging tile.  The last arriver re-zeroes the counter for the next launch.
__device__ __forceinline__ bool split_arrive(const SplitPart& sp, int* flag) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = atomicAdd(sp.cnt, 1);
        const int last = old == sp.split - 1;
        if (last) atomicExch(sp.cnt, 0);
        *flag = last;
    }
    __syncthreads();
    return *flag != 0;
}

// The rows part of one work item for a wavefront whose rows fill FMA 16-row blocks: the
// K loop into accumulators of exactly those blocks, then (after the workgroup barrier
// that frees the LDS stages) the activation and the bf16 rounding of its rows into the
// output staging tile.  Each variant owns its accumulators, so the register allocator
// never sees accumulators of one variant live in another.  Barriers: KT + 1, as in the
// DMA-only path of a wavefront without rows.
template <int BM, int NMAT, int ACT, int FMA>
__device__ __attribute__((always_inline)) inline bool rows_item(
    lds_char* lds, bf16_t* sC, int kt0, int KT, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb0,
    __amdgpu_buffer_rsrc_t rb1, const DmaPlan<LdsShape<BM, NMAT>::ADMA, LdsShape<BM, NMAT>::BDMA>& pl, int K,
    uint32_t rowB, int wave, int a_rd, int b_rd, int g, int wn, int rb, int wrows, int lq, int l16,
    const SplitPart& sp, int* flag) {
    using S = LdsShape<BM, NMAT>;
    constexpr int FN = S::FN, FO = (NMAT == 2) ? FN / 2 : FN, BNm = S::BNm, WTN = S::WTN;
    f32x4_t acc[FMA][FN];
#pragma unroll
    for (int i = 0; i < FMA; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc_zero(acc[i][j]);
    if constexpr (BM == 320) kloop_early<BM, NMAT, FMA>(lds, KT, ra, rb0, rb1, pl, K, rowB, wave, a_rd, b_rd, g, wn, acc, kt0);
    else kloop<BM, NMAT, FMA>(lds, KT, ra, rb0, rb1, pl, K, rowB, wave, a_rd, b_rd, g, wn, acc, kt0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the tail's zero loads land before LDS is reused
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const size_t wofs = (size_t)wave * S::FM * FN * 256 + lane * 4;
    // the item's part slots, and this part's byte offset within them (wavefront-uniform;
    // taken through readfirstlane so that the compiler keeps the descriptor in SGPRs)
    const uint64_t ib = (uint64_t)(uintptr_t)sp.item;
    const uint32_t ib_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)ib);
    const uint32_t ib_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(ib >> 32));
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(
        (const void*)(uintptr_t)(((uint64_t)ib_hi << 32) | ib_lo),
        (uint32_t)__builtin_amdgcn_readfirstlane((int)(sp.split * sp.slot_floats * 4)));
    const uint32_t pofs = (uint32_t)__builtin_amdgcn_readfirstlane((int)((sp.buf - sp.item) * 4));
    if (sp.buf) {
        // one part of a split item: store the accumulators (register layout, 16 bytes per
        // lane per block); the item's last part then reads all parts back in part order
        // (below), so its accumulators are not needed past this point
#pragma unroll
        for (int fm = 0; fm < FMA; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                store_part(rp, pofs + (uint32_t)((wofs + (size_t)(fm * FN + fn) * 256) * 4), acc[fm][fn]);
        if (!split_arrive(sp, flag)) return false;
    }
    // block (fm, fn) of the finished sums: the accumulators, or the parts added in order
    auto block = [&](int fm, int fn) -> f32x4_t {
        if (!sp.buf) return acc[fm][fn];
        const uint32_t o = (uint32_t)((wofs + (size_t)(fm * FN + fn) * 256) * 4);
        f32x4_t sum = load_part(rp, o);
        for (int q = 1; q < sp.split; ++q) sum += load_part(rp, o + (uint32_t)(q * sp.slot_floats * 4));
        return sum;
    };
#pragma unroll
    for (int fm = 0; fm < FMA; ++fm) {
        // only this wavefront's row blocks (with the even split of a 320-row tile, the
        // blocks past them are the other wavefront's rows)
        if (16 * fm >= wrows) break;
#pragma unroll
        for (int fo = 0; fo < FO; ++fo) {
            const int col = (NMAT == 2 ? wn * (BNm / S::WAVES_N) : wn * WTN) + 16 * fo + l16;
            const f32x4_t x = block(fm, fo);
            f32x4_t u = x;
            if constexpr (NMAT == 2) u = block(fm, fo + FN / 2);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float val = x[v];
                if constexpr (NMAT == 2) val = silu_f32(val) * u[v];
                else if constexpr (ACT == 1) val = silu_f32(val);
                const int r = rb + 16 * fm + 4 * lq + v;
                sC[r * S::CS_STRIDE + col] = f32_to_bf16(val);
            }
        }
    }
    return true;
}

// Wait until at most `pending` K steps' DMA of this wavefront are still in flight.
template <int DPW>
__device__ __forceinline__ void wait_dma(int pending) {
    if (pending >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * DPW) : "memory");
    else if (pending == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * DPW) : "memory");
    else if (pending == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DPW) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// All work items of one launch for row tiles of height BM (the persistent loop).
// part_buf / part_cnt: kPartSlots slots of BM x BN floats and kPartSlots counters (zero
// on entry) for the split of the last round, or NULL (no split).  Only the second
// projection splits: its K (the FFN width) is long, so a part's fp32 slot is small beside
// its operand stream; on the first projection (K = the model width) a split measured no
// faster, and the split's code alone made that kernel slower, so it is compiled out there.
template <int BM, int NMAT, int ACT, bool GATHER>
__device__ __forceinline__ void gemm_tiles(
    uint4* smem, const bf16_t* __restrict__ A, const int32_t* __restrict__ gather_rows,
    const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1, bf16_t* __restrict__ C,
    const Tile* __restrict__ tiles, const int32_t* __restrict__ ntiles_p, int K, int N,
    long long a_rows, float* __restrict__ part_buf, int* __restrict__ part_cnt) {
    using S = LdsShape<BM, NMAT>;
    constexpr int BNm = S::BNm, WAVES_N = S::WAVES_N, WTM = S::WTM, WTN = S::WTN, BK = S::BK;
    constexpr int FM = S::FM, FN = S::FN, ADMA = S::ADMA, BDMA = S::BDMA;
    constexpr int CS_STRIDE = S::CS_STRIDE, BROW = S::BROW;
    static_assert(ADMA >= 1 && BDMA >= 1, "every wavefront moves part of each operand");
    static_assert(NMAT == 1 || FN % 2 == 0, "SwiGLU wavefronts hold gate and up halves");

    lds_char* lds = (lds_char*)smem;
    bf16_t* sC = reinterpret_cast<bf16_t*>(smem);
    // the split parts' arrival flag: an LDS word past the output staging tile
    constexpr int FLAG_OFF = (BM * CS_STRIDE * 2 + 15) / 16 * 16;
    static_assert(FLAG_OFF + 16 <= (int)S::LDS_BYTES, "no LDS word left for the arrival flag");
    int* flag = reinterpret_cast<int*>(reinterpret_cast<char*>(smem) + FLAG_OFF);
    constexpr size_t SLOT = (size_t)BM * S::BN;       // floats per part slot
    static_assert(SLOT <= kGemmPartSlotFloats, "part slot larger than the workspace's");

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    const int NT = (N + BNm - 1) / BNm;
    const int KT = (K + BK - 1) / BK;
    const int ntiles = *ntiles_p;
    const long long total = (long long)ntiles * NT;
    const int G = gridDim.x;
    const long long first = (long long)(blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const uint32_t rowB = (uint32_t)N * 2;            // bytes per weight row in memory

    float* const pbuf = GATHER ? nullptr : part_buf;
    const WorkSplit wsp(total, G, pbuf ? KT : 0);
    for (long long w = first; w < wsp.nwork; w += G) {
        // per-lane constants, derived here from an opaque copy of the thread index: kept
        // live across the K loops they were spilled and reloaded at every item
        int tid_o = threadIdx.x;
        asm volatile("" : "+v"(tid_o));
        const int lane = tid_o & 63, l16 = lane & 15, lq = lane >> 4;
        // fragment read offsets: A row (wm*WTM + 16 fm + l16) chunk lq; W rows 8 lq + (l16 >> 2)
        const int a_rd = (wm * WTM + l16) * (BK * 2) + ((lq ^ swa4(l16)) << 4);
        // swizzle value of this lane's W rows (the same for rows k and k + 4 of its two reads)
        const int g = BM == 320 ? fk320<NMAT>(8 * lq + (l16 >> 2)) : ((l16 >> 2) & 3) | ((lq & 1) << 2);
        const int b_rd = (8 * lq + (l16 >> 2)) * BROW + (((l16 & 3) >> 1) << 4) + ((l16 & 1) << 3);
        // decode the work item (order: item_coords) and, for a split item, its part
        long long item;
        int part, slot;
        wsp.item_of(w, item, part, slot);
        // the item is the same for the whole workgroup: keep it (and what derives from it,
        // the tile, the operand resources) in scalar registers
        part = __builtin_amdgcn_readfirstlane(part);
        slot = __builtin_amdgcn_readfirstlane(slot);
        int mt, nt;
        item_coords(item, NT, tiles, mt, nt);
        mt = __builtin_amdgcn_readfirstlane(mt);
        nt = __builtin_amdgcn_readfirstlane(nt);
        const Tile tl = tiles[mt];
        const int rows = tl.row1 - tl.row0;
        const int n0 = nt * BNm;
        // K range of this work: all of K for an item of a complete round, else its part
        const int parts = slot >= 0 ? wsp.split : 1;
        const int kt0 = __builtin_amdgcn_readfirstlane((int)((long long)part * KT / parts));
        const int nsteps = __builtin_amdgcn_readfirstlane((int)((long long)(part + 1) * KT / parts) - kt0);
        SplitPart sp{nullptr, nullptr, nullptr, wsp.split, SLOT};
        if (pbuf && slot >= 0) {
            sp.item = pbuf + (size_t)slot * wsp.split * SLOT;
            sp.buf = sp.item + (size_t)part * SLOT;
            sp.cnt = part_cnt + slot;
        }
        // 320-row tiles split the tile's rows evenly between the two wavefront rows (at a
        // multiple of 16, so the A swizzle is unchanged): an expert with 256 rows then
        // multiplies 8 row blocks per wavefront instead of 10 and 6
        const int rsplit = BM == 320 ? min(WTM, (rows + 31) / 32 * 16) : WTM;
        const int rb = wm * rsplit;                   // this wavefront's first row
        const int wrows = min(rows - rb, rsplit);     // and its number of rows
        const bool wave_rows = wrows > 0;
        const int a_rd_item = a_rd + (rb - wm * WTM) * (BK * 2);

        DmaPlan<ADMA, BDMA> pl;
        // A: instruction i of this wavefront covers 16 rows x 4 chunks; lane -> (row, chunk)
#pragma unroll
        for (int i = 0; i < ADMA; ++i) {
            const int r = (wave * ADMA + i) * 16 + (lane >> 2);
            const int q = (lane & 3) ^ swa4(r);
            pl.a_k[i] = (uint32_t)(q * 8);
            long long row = tl.row0 + min(r, rows - 1);
            if constexpr (GATHER) row = gather_rows[row];
            else row -= tl.row0;
            // rows past the tile's own load nothing (zeros through the buffer bound)
            pl.a_off[i] = r < rows ? (uint32_t)(row * K * 2) + (uint32_t)(q * 16) : kOOB;
        }
        const __amdgpu_buffer_rsrc_t ra = GATHER ? make_rsrc(A, (uint32_t)(a_rows * K * 2))
                                                 : make_rsrc(A + (long long)tl.row0 * K, (uint32_t)rows * K * 2);
        const long long eoff = (long long)tl.e * K * N;
        const __amdgpu_buffer_rsrc_t rb0 = make_rsrc(B0 + eoff, (uint32_t)K * rowB);
        const __amdgpu_buffer_rsrc_t rb1 = make_rsrc((NMAT == 2 ? B1 : B0) + eoff, (uint32_t)K * rowB);
        // W: instruction j covers 2 rows x 32 chunks (SiLU2 / second projection) or
        // 4 rows x 16 chunks of one matrix (SwiGLU); for 320-row tiles, LDS bytes
        // [1024 j, 1024 j + 1024) of rows 384 (SiLU2) or 192 (SwiGLU, per matrix) bytes wide
#pragma unroll
        for (int i = 0; i < BDMA; ++i) {
            const int j = wave * BDMA + i;
            int k, c;
            if constexpr (BM == 320) {
                const int pos = (j % S::BMAT_DMA) * 1024 + lane * 16;   // byte within the matrix
                k = pos / BROW;
                c = ((pos % BROW) / 16) ^ (2 * fk320<NMAT>(k));
            } else if constexpr (NMAT == 1) {
                k = j * 2 + (lane >> 5);
                c = (lane & 31) ^ fk(k);
            } else {
                k = (j & 7) * 4 + (lane >> 4);
                c = (lane & 15) ^ fk(k);
            }
            const uint32_t col = (uint32_t)(n0 + 8 * c);
            // chunks past the tile's BNm columns (320-row tile) or past N are not loaded
            pl.b_off[i] = (8 * c < BNm && col < (uint32_t)N) ? (uint32_t)k * rowB + col * 2 : kOOB;
        }

        // prologue: the DMA ahead of the first step (steps past K read zeros, see kstep)
        dma_prologue<BM, NMAT>(lds, ra, rb0, rb1, pl, kt0, K, rowB, wave);
        bool write_out;       // the same in every wavefront of the workgroup
        if (wave_rows) {
            // a wavefront whose rows fill only the first blocks of its tile multiplies just
            // those (1, 2, 4, and for 320-row tiles 8 or 9 blocks of 16 rows, else all)
            const int ar = a_rd_item;
#define MOE_ROWS_ITEM(F_) rows_item<BM, NMAT, ACT, (F_)>(lds, sC, kt0, nsteps, ra, rb0, rb1, pl, K, rowB, wave, \
                                                           ar, b_rd, g, wn, rb, wrows, lq, l16, sp, flag)
            if (wrows <= 16) write_out = MOE_ROWS_ITEM(1);
            else if (FM > 2 && wrows <= 32) write_out = MOE_ROWS_ITEM(FM > 2 ? 2 : FM);
            else if (FM > 4 && wrows <= 64) write_out = MOE_ROWS_ITEM(FM > 4 ? 4 : FM);
            else if (BM == 320 && wrows <= 128) write_out = MOE_ROWS_ITEM(BM == 320 ? 8 : FM);
            else if (BM == 320 && wrows <= 144) write_out = MOE_ROWS_ITEM(BM == 320 ? 9 : FM);
            else write_out = MOE_ROWS_ITEM(FM);
#undef MOE_ROWS_ITEM
        } else {       // no rows for this wavefront: it still moves its share of the tiles
            for (int r = 0; r < nsteps; ++r) {
                wait_vmcnt<S::VMCNT>();
                kloop_barrier();
                dma_step<BM, NMAT>(lds, ra, rb0, rb1, pl, kt0, r, K, rowB, wave);
            }
            if constexpr (BM == 320) {      // the last barrier of kloop_early
                wait_vmcnt<S::VMCNT>();
                kloop_barrier();
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            write_out = sp.buf ? split_arrive(sp, flag) : true;
        }
        __syncthreads();
        constexpr int CPR = BNm / 8;
        for (int c = tid; write_out && c < rows * CPR; c += 256) {
            const int r = c / CPR, cc = c % CPR;
            const int col = n0 + cc * 8;
            if (col < N)
                __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(sC + r * CS_STRIDE + cc * 8),
                                            reinterpret_cast<u32x4_t*>(C + (long long)(tl.row0 + r) * N + col));
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // stores out before the next DMA count
        __syncthreads();
    }
}

// The grouped GEMM kernel.  BMA and BMB are the row-tile heights the tile list may use;
// the tile builder chose one from the actual per-expert counts and stored it in
// ntiles_p[1].  A single-height instance (BMA == BMB) returns at once when the list was
// built for another height (it is then the other half of a launch pair).
template <int BMA, int BMB>
struct LdsPair {
    template <int NMAT>
    static constexpr size_t bytes() {
        return LdsShape<BMA, NMAT>::LDS_BYTES > LdsShape<BMB, NMAT>::LDS_BYTES ? LdsShape<BMA, NMAT>::LDS_BYTES
                                                                               : LdsShape<BMB, NMAT>::LDS_BYTES;
    }
};

template <int BMA, int BMB, int NMAT, int ACT, bool GATHER>
__global__ __launch_bounds__(256, 1) void k_grouped_gemm_lds(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ gather_rows,
    const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1, bf16_t* __restrict__ C,
    const Tile* __restrict__ tiles, const int32_t* __restrict__ ntiles_p, int K, int N,
    long long a_rows, float* __restrict__ part_buf, int* __restrict__ part_cnt) {
    extern __shared__ uint4 smem[];
    const int bm = __builtin_amdgcn_readfirstlane(ntiles_p[1]);
    if (BMA == BMB && bm != BMA) return;      // the list is for the other kernel of the launch pair
    if (BMA != BMB && bm == BMB)
        gemm_tiles<BMB, NMAT, ACT, GATHER>(smem, A, gather_rows, B0, B1, C, tiles, ntiles_p, K, N, a_rows,
                                           part_buf, part_cnt);
    else
        gemm_tiles<BMA, NMAT, ACT, GATHER>(smem, A, gather_rows, B0, B1, C, tiles, ntiles_p, K, N, a_rows,
                                           part_buf, part_cnt);
}

// ------------------------------------------- ping-pong variant (two wavefront groups)
// Same tiles, LDS layout and DMA as above, with 8 wavefronts per workgroup in two groups
// of four (one wavefront of each group per SIMD, at most 128 accumulator registers each).
// Each group owns half the tile's rows; its four wavefronts split the columns.
// Each K step has a read phase (DMA issue and fragment reads) and an MFMA phase; the
// groups run them out of step, so one group's LDS reads and DMA issue overlap the other
// group's MFMAs.  Between two consecutive barriers one group is in its read phase and the
// other in its MFMA phase:
//   group 0:  R0 | M0 | R1 | M1 | ... | M(KT-1) | (idle)
//   group 1: (idle) | R0 | M0 | R1 | ... | R(KT-1) | M(KT-1)
// Both groups therefore pass 2 KT + 1 barriers per item (plus the prologue's).
//   * Step k is read in group 0's phase 2k and group 1's phase 2k+1.  Every wavefront
//     waits for its own DMA of step k before barrier 2k-1 (group 0 at the end of M(k-1),
//     group 1 at the end of R(k-1)), so all of step k has landed when it is read.
//   * R(k) starts the DMA of A for step k + NA - 1 and of W for step k + NW - 1, each into
//     the stage of its ring that held step k - 1.  Each read phase ends with lgkmcnt(0)
//     before its barrier, so both groups' reads of step k-1 (phases 2k-2 and 2k-1) are
//     complete before either group issues that DMA (phases 2k and 2k+1).
template <int BM, int NMAT>
struct PpShape {
    static constexpr int BN = BM == 320 ? 192 : 256, BNm = BN / NMAT, BK = 32;
    // W rows in LDS: 256 columns (512-byte rows, 16-byte chunk swizzle fk), or for 320-row
    // tiles the 192 columns they use (swizzle fk320), as in the 4-wavefront kernel
    static constexpr int LBN = BM == 320 ? 192 : 256, LBNm = LBN / NMAT;
    // ring depths: 320-row tiles stream their weights from HBM, 7 steps ahead
    static constexpr int NA = BM == 320 ? 3 : 4, NW = BM == 320 ? 8 : 4;
    static constexpr int GM = BM / 2;                        // rows of one group
    // A group's four wavefronts split its 128 x 256 tile by columns, 128 x 64 each: every
    // wavefront reads all the group's A rows (ds_read_b128) and a quarter of the W columns
    // (ds_read_b64_tr_b16, about half the rate per byte), so a K step costs the LDS some
    // 17% fewer clocks than with 64 x 128 tiles (2 x 2), at the same 128 accumulators.
    // 320-row tiles keep 2 x 2 (160 x 96).
    static constexpr int WCOLS = BM == 320 ? 2 : 4, WROWS = 4 / WCOLS;
    static constexpr int WTM = GM / WROWS, WTN = BN / WCOLS; // wavefront tile
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static constexpr int A_STAGE = BM * BK * 2, B_STAGE = BK * LBN * 2;
    static constexpr int W_RING = NA * A_STAGE;              // LDS offset of the W ring
    static constexpr int A_INSTR = A_STAGE / 1024, B_INSTR = B_STAGE / 1024;
    static constexpr int BMAT_DMA = B_INSTR / NMAT;          // W instructions per matrix
    // A instruction j goes to wavefront j % 8: group 0 (wavefronts 0-3) may take one more.
    // W instructions: BDMA0 per group-0 wavefront, then BDMA1 per group-1 wavefront, so
    // that both groups issue DPW instructions per step.
    static constexpr int ADMA0 = (A_INSTR + 7 - 0) / 8, ADMA1 = (A_INSTR + 7 - 4) / 8;
    static constexpr int DPW = (A_INSTR + B_INSTR) / 8;
    static constexpr int BDMA0 = DPW - ADMA0, BDMA1 = DPW - ADMA1;
    static constexpr int BROW = 2 * LBNm, CS_STRIDE = BNm + 8;
    // the wait before a step, per group: see LdsShape::VMCNT
    template <int GROUP>
    static constexpr int vmcnt() {
        return NW > NA ? (GROUP == 0 ? BDMA0 : BDMA1) + (NA - 2) * DPW : (NW - 2) * DPW;
    }
    // the split parts' arrival flag: an LDS word past the output staging tile
    static constexpr int FLAG_OFF = (BM * CS_STRIDE * 2 + 15) / 16 * 16;
    static constexpr size_t RING_BYTES = (size_t)NA * A_STAGE + (size_t)NW * B_STAGE;
    static constexpr size_t LDS_BYTES = RING_BYTES > (size_t)FLAG_OFF + 16 ? RING_BYTES : (size_t)FLAG_OFF + 16;
    static_assert(A_INSTR % 8 == 0 || A_INSTR % 8 == 4, "A instructions split by groups");
    static_assert((A_INSTR + B_INSTR) % 8 == 0 && BDMA0 >= 1 && BDMA1 >= 1, "DMA split evenly by wavefronts");
    static_assert(4 * BDMA0 + 4 * BDMA1 == B_INSTR, "every W instruction has a wavefront");
    static_assert(NW >= NA && NA >= 2 && (NW - 1) * DPW < 64, "ring depths");
};

template <int ADMA, int BDMA>
struct PpPlan {
    uint32_t a_off[ADMA], a_k[ADMA], b_off[BDMA];
};

template <int BM, int NMAT, int GROUP>
using PpPlanOf = PpPlan<GROUP == 0 ? PpShape<BM, NMAT>::ADMA0 : PpShape<BM, NMAT>::ADMA1,
                        GROUP == 0 ? PpShape<BM, NMAT>::BDMA0 : PpShape<BM, NMAT>::BDMA1>;

// First W instruction of a wavefront (wavefronts of group 0 take BDMA0 each, then group 1).
template <int BM, int NMAT, int GROUP>
__device__ __forceinline__ int pp_w_first(int wave) {
    using S = PpShape<BM, NMAT>;
    return GROUP == 0 ? wave * S::BDMA0 : 4 * S::BDMA0 + (wave - 4) * S::BDMA1;
}

// This wavefront's share of the A DMA of K step kt into A stage `dst` (`dummy`: zeros).
template <int BM, int NMAT, int GROUP>
__device__ __forceinline__ void pp_dma_a(lds_char* dst, __amdgpu_buffer_rsrc_t ra,
                                         const PpPlanOf<BM, NMAT, GROUP>& pl, int kt, int K, int wave,
                                         bool dummy = false) {
    using S = PpShape<BM, NMAT>;
    constexpr int ADMA = GROUP == 0 ? S::ADMA0 : S::ADMA1;
    const uint32_t k0 = (uint32_t)kt * S::BK;
#pragma unroll
    for (int i = 0; i < ADMA; ++i) {
        const uint32_t off = (!dummy && k0 + pl.a_k[i] < (uint32_t)K) ? pl.a_off[i] + k0 * 2 : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(dst + (wave + 8 * i) * 1024), 16, off, 0, 0, 0);
    }
}

// This wavefront's share of the W DMA of K step kt into W stage `dst`, with cache policy
// WAUX (kWStream: the non-temporal hint, for a slice that one work item reads).
template <int BM, int NMAT, int GROUP, int WAUX>
__device__ __forceinline__ void pp_dma_w(lds_char* dst, __amdgpu_buffer_rsrc_t rb0, __amdgpu_buffer_rsrc_t rb1,
                                         const PpPlanOf<BM, NMAT, GROUP>& pl, int kt, uint32_t rowB, int wave) {
    using S = PpShape<BM, NMAT>;
    constexpr int BDMA = GROUP == 0 ? S::BDMA0 : S::BDMA1;
    const uint32_t k0 = (uint32_t)kt * S::BK;
    const int j0 = pp_w_first<BM, NMAT, GROUP>(wave);
#pragma unroll
    for (int i = 0; i < BDMA; ++i) {
        const int j = j0 + i;
        const uint32_t off = pl.b_off[i] == kOOB ? kOOB : pl.b_off[i] + k0 * rowB;
        const __amdgpu_buffer_rsrc_t rb = (NMAT == 2 && j >= S::BMAT_DMA) ? rb1 : rb0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(dst + j * 1024), 16, off, 0, 0, WAUX);
    }
}

// One read phase's DMA: A of step r + NA - 1 and W of step r + NW - 1 (r relative to the
// work's first step kt0), each into the stage its ring held for step r - 1.
template <int BM, int NMAT, int GROUP, int WAUX>
__device__ __forceinline__ void pp_dma_step(lds_char* lds, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb0,
                                            __amdgpu_buffer_rsrc_t rb1, const PpPlanOf<BM, NMAT, GROUP>& pl,
                                            int kt0, int r, int K, uint32_t rowB, int wave) {
    using S = PpShape<BM, NMAT>;
    const int ra_step = r + S::NA - 1, rw_step = r + S::NW - 1;
    pp_dma_a<BM, NMAT, GROUP>(lds + (ra_step % S::NA) * S::A_STAGE, ra, pl, kt0 + ra_step, K, wave);
    pp_dma_w<BM, NMAT, GROUP, WAUX>(lds + S::W_RING + (rw_step % S::NW) * S::B_STAGE, rb0, rb1, pl, kt0 + rw_step,
                              rowB, wave);
}

// DMA plan of one wavefront for one tile: A instruction j = wave + 8 i covers 16 rows x
// 4 chunks; W instruction j (from pp_w_first) is placed as in the 4-wavefront kernel.
template <int BM, int NMAT, int GROUP, bool GATHER>
__device__ __forceinline__ void pp_plan(PpPlanOf<BM, NMAT, GROUP>& pl, const Tile& tl, int rows, int n0, int K,
                                        int N, const int32_t* __restrict__ gather_rows, int wave, int lane) {
    using S = PpShape<BM, NMAT>;
    constexpr int ADMA = GROUP == 0 ? S::ADMA0 : S::ADMA1, BDMA = GROUP == 0 ? S::BDMA0 : S::BDMA1;
    const uint32_t rowB = (uint32_t)N * 2;
#pragma unroll
    for (int i = 0; i < ADMA; ++i) {
        const int r = (wave + 8 * i) * 16 + (lane >> 2);
        const int q = (lane & 3) ^ swa4(r);
        pl.a_k[i] = (uint32_t)(q * 8);
        long long row = tl.row0 + min(r, rows - 1);
        if constexpr (GATHER) row = gather_rows[row];
        else row -= tl.row0;
        pl.a_off[i] = r < rows ? (uint32_t)(row * K * 2) + (uint32_t)(q * 16) : kOOB;
    }
    const int j0 = pp_w_first<BM, NMAT, GROUP>(wave);
#pragma unroll
    for (int i = 0; i < BDMA; ++i) {
        const int j = j0 + i;
        int k, c;
        if constexpr (BM == 320) {
            const int pos = (j % S::BMAT_DMA) * 1024 + lane * 16;   // byte within the matrix
            k = pos / S::BROW;
            c = ((pos % S::BROW) / 16) ^ (2 * fk320<NMAT>(k));
        } else if constexpr (NMAT == 1) {
            k = j * 2 + (lane >> 5);
            c = (lane & 31) ^ fk(k);
        } else {
            k = (j & 7) * 4 + (lane >> 4);
            c = (lane & 15) ^ fk(k);
        }
        const uint32_t col = (uint32_t)(n0 + 8 * c);
        pl.b_off[i] = (8 * c < S::BNm && col < (uint32_t)N) ? (uint32_t)k * rowB + col * 2 : kOOB;
    }
}

template <int BM, int NMAT>
__device__ __forceinline__ void pp_read(const lds_char* As, const lds_char* Bs, int a_rd, int b_rd, int g, int wn,
                                        bf16x8_t (&af)[PpShape<BM, NMAT>::FM],
                                        bf16x8_t (&bfr)[PpShape<BM, NMAT>::FN]) {
    using S = PpShape<BM, NMAT>;
    constexpr int FM = S::FM, FN = S::FN, BROW = S::BROW;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
        af[fm] = *(const __attribute__((address_space(3))) bf16x8_t*)(As + a_rd + fm * 16 * S::BK * 2);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        int mat, blk;
        if constexpr (NMAT == 1) {
            mat = 0;
            blk = wn * (S::WTN / 16) + fn;
        } else {
            mat = fn < FN / 2 ? 0 : 1;
            blk = wn * (FN / 2) + (fn % (FN / 2));
        }
        const lds_char* p = Bs + mat * S::BK * BROW + b_rd + (wblk<BM, NMAT>(blk, g) << 5);
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)p);
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(p + 4 * BROW));
        const v8i16_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        bfr[fn] = __builtin_bit_cast(bf16x8_t, v);
    }
}

// The K loop of one group (see the phase table above) over K steps kt0 .. kt0 + KT - 1.
// `nblk`: the wavefront's 16-row blocks that hold rows of the tile (only they are
// multiplied; with none the wavefront only moves its DMA share and keeps the barriers).
template <int GROUP, int BM, int NMAT, int WAUX>
__device__ __attribute__((always_inline)) inline void pp_kloop(
    lds_char* lds, int kt0, int KT, int nblk, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb0,
    __amdgpu_buffer_rsrc_t rb1, const PpPlanOf<BM, NMAT, GROUP>& pl, int K, uint32_t rowB, int wave, int a_rd,
    int b_rd, int g, int wn, f32x4_t (&acc)[PpShape<BM, NMAT>::FM][PpShape<BM, NMAT>::FN]) {
    using S = PpShape<BM, NMAT>;
    constexpr int FM = S::FM, FN = S::FN, VMCNT = S::template vmcnt<GROUP>();
    bf16x8_t af[FM], bfr[FN];
    if constexpr (GROUP == 1) kloop_barrier();                  // group 1's idle first phase
    for (int kt = 0; kt < KT; ++kt) {
        // read phase: fragments of step kt, then the DMA of the steps NA - 1 and NW - 1 ahead
        // (read by every wavefront: a branch here makes the compiler copy the fragments)
        pp_read<BM, NMAT>(lds + (kt % S::NA) * S::A_STAGE, lds + S::W_RING + (kt % S::NW) * S::B_STAGE, a_rd, b_rd,
                          g, wn, af, bfr);
        __builtin_amdgcn_sched_barrier(0);
        pp_dma_step<BM, NMAT, GROUP, WAUX>(lds, ra, rb0, rb1, pl, kt0, kt, K, rowB, wave);
        wait_lgkm0();
        if constexpr (GROUP == 1) wait_vmcnt<VMCNT>();           // step kt + 1 complete
        kloop_barrier();
        // MFMA phase (the guards are laid out as fall-throughs: a full tile takes no branch;
        // with the compiler's own layout it took two or three per step)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            if (__builtin_expect(fm < nblk, 1)) {
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
            }
        }
        // the accumulators live in AGPRs (at two wavefronts per SIMD the compiler would
        // otherwise keep them in VGPRs, next to the fragments, and spill)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) asm volatile("" : "+a"(acc[fm][fn]));
        if constexpr (GROUP == 0) wait_vmcnt<VMCNT>();           // step kt + 1 complete
        kloop_barrier();
    }
    if constexpr (GROUP == 0) kloop_barrier();                  // group 0's idle last phase
}

// The whole K loop of one work item for group GROUP: plan, prologue, loop.  The prologue
// issues the DMA as the steps -(NW - 1) .. -1 would have (A of steps below 0 as zero
// placeholders), so the first steps wait with the same count as the rest.  WAUX: the
// cache policy of the W loads.
template <int GROUP, int BM, int NMAT, bool GATHER, int WAUX>
__device__ __attribute__((always_inline)) inline void pp_item(
    lds_char* lds, int kt0, int KT, int nblk, const Tile& tl, int rows, int n0, int K, int N,
    __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb0, __amdgpu_buffer_rsrc_t rb1,
    const int32_t* __restrict__ gather_rows, int wave, int lane, int a_rd, int b_rd, int g, int wn,
    f32x4_t (&acc)[PpShape<BM, NMAT>::FM][PpShape<BM, NMAT>::FN]) {
    using S = PpShape<BM, NMAT>;
    const uint32_t rowB = (uint32_t)N * 2;
    PpPlanOf<BM, NMAT, GROUP> pl;
    pp_plan<BM, NMAT, GROUP, GATHER>(pl, tl, rows, n0, K, N, gather_rows, wave, lane);
#pragma unroll
    for (int r = -(S::NW - 1); r < 0; ++r) {
        const int ra_step = r + S::NA - 1, rw_step = r + S::NW - 1;
        const int aslot = ((ra_step % S::NA) + S::NA) % S::NA;
        pp_dma_a<BM, NMAT, GROUP>(lds + aslot * S::A_STAGE, ra, pl, kt0 + ra_step, K, wave, ra_step < 0);
        pp_dma_w<BM, NMAT, GROUP, WAUX>(lds + S::W_RING + rw_step * S::B_STAGE, rb0, rb1, pl, kt0 + rw_step, rowB, wave);
    }
    wait_vmcnt<S::template vmcnt<GROUP>()>();                    // step 0 complete for all
    kloop_barrier();
    pp_kloop<GROUP, BM, NMAT, WAUX>(lds, kt0, KT, nblk, ra, rb0, rb1, pl, K, rowB, wave, a_rd, b_rd, g, wn, acc);
}

// Output of one ping-pong work item: block(fm, fn) gives this wavefront's fp32 sums for
// accumulator block (fm, fn); the activation is applied, rounded to bf16 and staged in LDS
// (the K loop's stages are free by then), then written out as 16-byte row pieces.
// C_rows: the item's first output row.
template <int BM, int NMAT, int ACT, typename BlockFn>
__device__ __forceinline__ void pp_write_out(lds_char* lds, BlockFn block, int nblk, int row0, int wn,
                                             int l16, int lq, int tid, int rows, int n0, int N,
                                             bf16_t* __restrict__ C_rows) {
    using S = PpShape<BM, NMAT>;
    constexpr int FM = S::FM, FN = S::FN, BNm = S::BNm, WTN = S::WTN, CS_STRIDE = S::CS_STRIDE;
    constexpr int FO = (NMAT == 2) ? FN / 2 : FN;
    typedef __attribute__((address_space(3))) bf16_t lds_bf16;
    lds_bf16* sC = reinterpret_cast<lds_bf16*>(lds);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        if (fm >= nblk) break;                 // blocks past the wavefront's rows
#pragma unroll
        for (int fo = 0; fo < FO; ++fo) {
            const int col = wn * (WTN / NMAT) + 16 * fo + l16;
            const f32x4_t x = block(fm, fo);
            f32x4_t u = x;
            if constexpr (NMAT == 2) u = block(fm, fo + FN / 2);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float val = x[v];
                if constexpr (NMAT == 2) val = silu_f32(val) * u[v];
                else if constexpr (ACT == 1) val = silu_f32(val);
                const int r = row0 + 16 * fm + 4 * lq + v;
                sC[r * CS_STRIDE + col] = f32_to_bf16(val);
            }
        }
    }
    __syncthreads();
    constexpr int CPR = BNm / 8;
    for (int c = tid; c < rows * CPR; c += 512) {
        const int r = c / CPR, cc = c % CPR;
        const int col = n0 + cc * 8;
        if (col < N)
            __builtin_nontemporal_store(
                *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(sC + r * CS_STRIDE + cc * 8),
                reinterpret_cast<u32x4_t*>(C_rows + (long long)r * N + col));
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

// The output of a split item's last part: the parts' sums, added in part order, through
// pp_write_out.  Kept out of line so that the split tail's registers do not weigh on the
// allocation of the kernel's K loops.
template <int BM, int NMAT, int ACT>
__device__ __attribute__((noinline)) void pp_write_split(lds_char* lds, __amdgpu_buffer_rsrc_t rp, uint32_t wofs,
                                                         int nsplit, int nblk, int row0, int wn, int l16,
                                                         int lq, int tid, int rows, int n0, int N,
                                                         bf16_t* __restrict__ C_rows) {
    using S = PpShape<BM, NMAT>;
    constexpr int FN = S::FN;
    constexpr uint32_t SLOT_BYTES = (uint32_t)BM * S::BN * 4;
    auto block = [&](int fm, int fn) -> f32x4_t {
        const uint32_t o = wofs + (uint32_t)((fm * FN + fn) * 1024);
        f32x4_t sum = load_part(rp, o);
        for (int q = 1; q < nsplit; ++q) sum += load_part(rp, o + (uint32_t)q * SLOT_BYTES);
        return sum;
    };
    pp_write_out<BM, NMAT, ACT>(lds, block, nblk, row0, wn, l16, lq, tid, rows, n0, N, C_rows);
}

// ------------------------------------------ thin row tiles inside the ping-pong kernel
// A row tile of at most 64 rows (an expert with few rows, or the ragged last tile of a
// long one) does little MFMA work: its cost is streaming its weight slice.  The ping-pong
// K loop would spend on it what it spends on a full tile: two phases and four barriers
// per K step, every wavefront reading all its fragments, and 16 A loads per step of which
// most only write zeros.  Such a tile instead runs this loop: one barrier per K step, an
// A stage of 64 rows (4 loads), both operands in rings of ThinShape::NS stages with the
// DMA LEAD steps ahead (more weight bytes in flight per CU), and each wavefront
// multiplying only the 16-row blocks that hold rows, for its own output columns: 16 of
// them (gate and up) for SwiGLU, else 32.  The LDS layouts and swizzles are those of the
// 256-row tile (W rows of 256 columns, A rows of 64 bytes), so the fragment reads are the
// ping-pong kernel's.
template <int NMAT>
struct ThinShape {
    using P = PpShape<256, NMAT>;
    static constexpr int BK = 32, ROWS = 64;
    static constexpr int A_STAGE = ROWS * BK * 2;           // 4 KB
    static constexpr int B_STAGE = P::B_STAGE;              // 16 KB: 32 rows x 256 columns
    static constexpr int NS = 8, LEAD = NS - 1;             // stages per operand, DMA lead
    static constexpr int W_RING = 0, A_RING = NS * B_STAGE;
    static constexpr int AINSTR = A_STAGE / 1024;           // A loads per step: wavefronts 0-3
    static constexpr int BINSTR = B_STAGE / 1024;           // W loads per step: 2 per wavefront
    static constexpr int RING_BYTES = NS * (A_STAGE + B_STAGE);
    static_assert(RING_BYTES <= 160 * 1024, "the thin rings fit the LDS");
    static_assert(BINSTR == 16 && AINSTR == 4, "wavefront w loads W pieces 2w, 2w + 1 and A piece w < 4");
    static_assert((LEAD - 1) * 3 < 64, "DMA in flight fits the 6-bit vmcnt");
};

// LDS of a ping-pong launch: its rings (or the output staging tile) and the thin tiles' rings.
template <int BM, int NMAT>
constexpr size_t pp_lds_bytes() {
    return BM == 256 && (size_t)ThinShape<NMAT>::RING_BYTES > PpShape<BM, NMAT>::LDS_BYTES
               ? (size_t)ThinShape<NMAT>::RING_BYTES
               : PpShape<BM, NMAT>::LDS_BYTES;
}

// One K step of a thin tile: the DMA of step s + LEAD into the stages `dA` / `dB` (those
// of step s - 1), then this step's fragments from `As` / `Bs` and its MFMAs.  The stages
// are distinct, and saying so with __restrict__ lets the compiler issue the fragment reads
// without waiting for the DMA in flight.
template <int NMAT, int WAUX>
__device__ __attribute__((always_inline)) inline void thin_step(
    const lds_char* __restrict__ As, const lds_char* __restrict__ Bs, lds_char* __restrict__ dA,
    lds_char* __restrict__ dB, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, uint32_t a_off, uint32_t a_k,
    const uint32_t (&b_off)[2], uint32_t k0, int K, uint32_t rowB, int wave, int a_rd, int b_rd, int g, int blk0,
    int mat1, int blk1, int fmt, f32x4_t (&acc)[4][2]) {
    using S = ThinShape<NMAT>;
    using P = PpShape<256, NMAT>;
    constexpr int BK = S::BK, BROW = P::BROW;
    if (wave < S::AINSTR) {
        const uint32_t off = (k0 + a_k < (uint32_t)K) ? a_off + k0 * 2 : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(dA + wave * 1024), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t off = (k0 >= (uint32_t)K || b_off[i] == kOOB) ? kOOB : b_off[i] + k0 * rowB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(dB + (2 * wave + i) * 1024), 16, off, 0, 0, WAUX);
    }
    auto read_b = [&](int mat, int blk) -> bf16x8_t {
        const lds_char* p = Bs + mat * BK * BROW + b_rd + (wblk<256, NMAT>(blk, g) << 5);
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)p);
        const v4i16_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(p + 4 * BROW));
        const v8i16_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8_t, v);
    };
    const bf16x8_t b0 = read_b(0, blk0), b1 = read_b(mat1, blk1);
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) {
        if (fm < fmt) {
            const bf16x8_t a = *(const __attribute__((address_space(3))) bf16x8_t*)(As + a_rd + fm * 16 * BK * 2);
            acc[fm][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b0, acc[fm][0], 0, 0, 0);
            acc[fm][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, acc[fm][1], 0, 0, 0);
        }
    }
}

// The whole thin tile: plan, prologue, K loop, epilogue.  Every value that selects memory
// (the tile, the operand resources) is wavefront-uniform and kept in scalar registers.
template <int NMAT, int ACT, bool GATHER, int WAUX, typename Claim>
__device__ __attribute__((always_inline)) inline void pp_thin_item(
    lds_char* lds, const bf16_t* __restrict__ A, long long a_rows, const int32_t* __restrict__ gather_rows,
    const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1, bf16_t* __restrict__ C, int e, int row0, int rows,
    int n0, int K, int N, Claim&& claim) {
    using S = ThinShape<NMAT>;
    using P = PpShape<256, NMAT>;
    constexpr int BK = S::BK, BROW = P::BROW, BNm = P::BNm, CS_STRIDE = P::CS_STRIDE, NS = S::NS, LEAD = S::LEAD;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lq = lane >> 4;
    const int KT = (K + BK - 1) / BK;
    const uint32_t rowB = (uint32_t)N * 2;
    const __amdgpu_buffer_rsrc_t ra = GATHER ? make_rsrc(A, (uint32_t)(a_rows * K * 2))
                                             : make_rsrc(A + (long long)row0 * K, (uint32_t)rows * K * 2);
    const long long eoff = (long long)e * K * N;
    // W piece j = 2 wave + i; SwiGLU's pieces 8..15 are the up matrix's
    const __amdgpu_buffer_rsrc_t rb = make_rsrc((NMAT == 2 && wave >= 4 ? B1 : B0) + eoff, (uint32_t)K * rowB);
    // A piece `wave` (wavefronts 0-3): rows 16 wave .. 16 wave + 15, four 16-byte chunks each
    uint32_t a_off = kOOB, a_k = 0;
    if (wave < S::AINSTR) {
        const int r = wave * 16 + (lane >> 2);
        const int q = (lane & 3) ^ swa4(r);
        a_k = (uint32_t)(q * 8);
        long long row = row0 + min(r, rows - 1);
        if constexpr (GATHER) row = gather_rows[row];
        else row -= row0;
        a_off = r < rows ? (uint32_t)(row * K * 2) + (uint32_t)(q * 16) : kOOB;
    }
    // W pieces, placed as in the 256-row tile
    uint32_t b_off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int j = 2 * wave + i;
        int k, c;
        if constexpr (NMAT == 1) {
            k = j * 2 + (lane >> 5);
            c = (lane & 31) ^ fk(k);
        } else {
            k = (j & 7) * 4 + (lane >> 4);
            c = (lane & 15) ^ fk(k);
        }
        const uint32_t col = (uint32_t)(n0 + 8 * c);
        b_off[i] = (8 * c < BNm && col < (uint32_t)N) ? (uint32_t)k * rowB + col * 2 : kOOB;
    }
    // fragment reads (the ping-pong kernel's addressing for the 256-row tile)
    const int a_rd = l16 * (BK * 2) + ((lq ^ swa4(l16)) << 4);
    const int g = ((l16 >> 2) & 3) | ((lq & 1) << 2);
    const int b_rd = (8 * lq + (l16 >> 2)) * BROW + (((l16 & 3) >> 1) << 4) + ((l16 & 1) << 3);
    // this wavefront's two column blocks: SwiGLU gate / up block `wave`, else blocks 2 wave, 2 wave + 1
    const int mat1 = NMAT == 2 ? 1 : 0;
    const int blk0 = NMAT == 2 ? wave : 2 * wave, blk1 = NMAT == 2 ? wave : 2 * wave + 1;
    const int fmt = __builtin_amdgcn_readfirstlane((rows + 15) / 16);   // row blocks holding rows (1..4)
    f32x4_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[i][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        acc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // prologue: the DMA of steps 0 .. LEAD - 1 into stages 0 .. LEAD - 1
#pragma unroll
    for (int s = 0; s < LEAD; ++s) {
        const uint32_t k0 = (uint32_t)s * BK;
        if (wave < S::AINSTR) {
            const uint32_t off = (k0 + a_k < (uint32_t)K) ? a_off + k0 * 2 : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (lds_void*)(lds + S::A_RING + s * S::A_STAGE + wave * 1024), 16, off, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t off = (k0 >= (uint32_t)K || b_off[i] == kOOB) ? kOOB : b_off[i] + k0 * rowB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (lds_void*)(lds + S::W_RING + s * S::B_STAGE + (2 * wave + i) * 1024), 16, off, 0, 0, WAUX);
        }
    }
    for (int s = 0; s < KT; ++s) {
        // this wavefront's DMA of step s has landed (LEAD - 1 later steps may be in flight),
        // and its fragment reads of step s - 1 are done; after the barrier both hold for all
        if (wave < S::AINSTR) wait_vmcnt<(LEAD - 1) * 3>();
        else wait_vmcnt<(LEAD - 1) * 2>();
        wait_lgkm0();
        kloop_barrier();
        const int cur = s % NS, nxt = (s + LEAD) % NS;       // nxt: the stage step s - 1 used
        thin_step<NMAT, WAUX>(lds + S::A_RING + cur * S::A_STAGE, lds + S::W_RING + cur * S::B_STAGE,
                              lds + S::A_RING + nxt * S::A_STAGE, lds + S::W_RING + nxt * S::B_STAGE, ra, rb,
                              a_off, a_k, b_off, (uint32_t)(s + LEAD) * BK, K, rowB, wave, a_rd, b_rd, g, blk0, mat1,
                              blk1, fmt, acc);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the zero loads past K land before LDS is reused
    __syncthreads();
    claim();                                            // the next work item, during the epilogue
    // epilogue: activation, one rounding to bf16, staged in LDS, written as 16-byte row pieces
    typedef __attribute__((address_space(3))) bf16_t lds_bf16;
    lds_bf16* sC = reinterpret_cast<lds_bf16*>(lds);
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) {
        if (fm >= fmt) break;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * fm + 4 * lq + v;
            if constexpr (NMAT == 2) {
                sC[r * CS_STRIDE + 16 * wave + l16] = f32_to_bf16(silu_f32(acc[fm][0][v]) * acc[fm][1][v]);
            } else {
                float v0 = acc[fm][0][v], v1 = acc[fm][1][v];
                if constexpr (ACT == 1) {
                    v0 = silu_f32(v0);
                    v1 = silu_f32(v1);
                }
                sC[r * CS_STRIDE + 32 * wave + l16] = f32_to_bf16(v0);
                sC[r * CS_STRIDE + 32 * wave + 16 + l16] = f32_to_bf16(v1);
            }
        }
    }
    __syncthreads();
    constexpr int CPR = BNm / 8;
    bf16_t* C_rows = C + (long long)row0 * N;
    for (int c = tid; c < rows * CPR; c += 512) {
        const int r = c / CPR, cc = c % CPR;
        const int col = n0 + cc * 8;
        if (col < N)
            __builtin_nontemporal_store(
                *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(sC + r * CS_STRIDE + cc * 8),
                reinterpret_cast<u32x4_t*>(C_rows + (long long)r * N + col));
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

// All work items of one launch, ping-pong form.  part_buf / part_cnt as for gemm_tiles
// (the split of the last round), used by the SPLIT instance only.
template <int BM, int NMAT, int ACT, bool GATHER, bool SPLIT>
__device__ __forceinline__ void gemm_tiles_pp(
    uint4* smem, const bf16_t* __restrict__ A, const int32_t* __restrict__ gather_rows,
    const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1, bf16_t* __restrict__ C,
    const Tile* __restrict__ tiles, const int32_t* __restrict__ ntiles_p, int K, int N,
    long long a_rows, float* __restrict__ part_buf, int* __restrict__ part_cnt, int* __restrict__ item_q) {
    using S = PpShape<BM, NMAT>;
    constexpr int BNm = S::BNm, GM = S::GM, WTM = S::WTM, WTN = S::WTN, BK = S::BK;
    constexpr int FM = S::FM, FN = S::FN, BROW = S::BROW;
    static_assert(NMAT == 1 || FN % 2 == 0, "SwiGLU wavefronts hold gate and up halves");
    constexpr size_t SLOT = (size_t)BM * S::BN;       // floats per part slot
    static_assert(SLOT <= kGemmPartSlotFloats, "part slot larger than the workspace's");
    static_assert(8 * FM * FN * 256 == (int)SLOT, "eight wavefronts' accumulators fill a slot");
    lds_char* lds = (lds_char*)smem;
    bf16_t* sC = reinterpret_cast<bf16_t*>(smem);
    int* flag = reinterpret_cast<int*>(reinterpret_cast<char*>(smem) + S::FLAG_OFF);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, wsub = (wave & 3) / S::WCOLS, wn = wave % S::WCOLS;
    const int wr = S::WROWS * grp + wsub;                        // this wavefront's row piece

    const int NT = (N + BNm - 1) / BNm;
    const int KT = (K + BK - 1) / BK;
    const long long total = (long long)(*ntiles_p) * NT;
    const int G = gridDim.x;
    const long long first = (long long)(blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const uint32_t rowB = (uint32_t)N * 2;

    static_assert(!(SPLIT && GATHER), "only the second projection splits");
    float* const pbuf = SPLIT ? part_buf : nullptr;

    // Work queues (item_q; the work order below).  Thread 0 claims the next work item from
    // its XCD's queue once the current item's K loop is done (cn), so the atomic's latency
    // passes during the epilogue.
    const int xcd = blockIdx.x & 7, per_xcd = G >> 3;
    int cn = 0;
    auto claim = [&]() __attribute__((always_inline)) {
        if (item_q && tid == 0) cn = atomicAdd(item_q + xcd, 1);
    };

    // One work item: the whole K range (PART false), or part `part` of `nsplit` of the item
    // whose parts use slot `slot` of the part buffer.  The full rounds and the split tail run
    // in loops of their own, so the full rounds carry none of the split's state in registers.
    auto run_item = [&](long long item, int part, int nsplit, int slot, auto split_tag)
                        __attribute__((always_inline)) {
        constexpr bool PART = decltype(split_tag)::value;
        // per-lane constants, derived here from an opaque copy of the thread index: kept
        // live across the K loops they were spilled, and reloading them cost every item
        // some 5k cycles of serialized scratch reads
        int tid_o = threadIdx.x;
        asm volatile("" : "+v"(tid_o));
        const int lane = tid_o & 63, l16 = lane & 15, lq = lane >> 4;
        // A fragment reads at row 0 of the wavefront's rows (the rows move per item, by
        // multiples of 16, which keep the A swizzle)
        const int a_rd0 = l16 * (BK * 2) + ((lq ^ swa4(l16)) << 4);
        // swizzle value of this lane's W rows (the same for rows k and k + 4 of its two reads)
        const int g = BM == 320 ? fk320<NMAT>(8 * lq + (l16 >> 2)) : ((l16 >> 2) & 3) | ((lq & 1) << 2);
        const int b_rd = (8 * lq + (l16 >> 2)) * BROW + (((l16 & 3) >> 1) << 4) + ((l16 & 1) << 3);
        int mt, nt;
        item_coords(item, NT, tiles, mt, nt);
        mt = __builtin_amdgcn_readfirstlane(mt);
        nt = __builtin_amdgcn_readfirstlane(nt);
        const Tile tl = tiles[mt];
        const int rows = tl.row1 - tl.row0;
        const int n0 = nt * BNm;
        if constexpr (!PART && BM == 256) {
            if (rows <= ThinShape<NMAT>::ROWS) {      // a thin tile: its own loop
                if (tl.cnt == 1)
                    pp_thin_item<NMAT, ACT, GATHER, kWStream>(lds, A, a_rows, gather_rows, B0, B1, C, tl.e, tl.row0,
                                                              rows, n0, K, N, claim);
                else
                    pp_thin_item<NMAT, ACT, GATHER, 0>(lds, A, a_rows, gather_rows, B0, B1, C, tl.e, tl.row0, rows,
                                                       n0, K, N, claim);
                return;
            }
        }
        // the tile's rows split evenly over the row pieces (one per group; two per group for
        // 320-row tiles), at a multiple of 16 (an expert with 256 rows in a 320-row tile
        // multiplies 4 row blocks per wavefront, not 5, 5, 5 and 1)
        constexpr int NPIECE = 2 * S::WROWS;
        const int rsplit = min(WTM, (rows + 16 * NPIECE - 1) / (16 * NPIECE) * 16);
        const int row0 = wr * rsplit;                            // first tile row of this wavefront
        const int wrows = min(rows - row0, rsplit);
        const int nblk = wrows > 0 ? (wrows + 15) / 16 : 0;
        const int a_rd = a_rd0 + row0 * (BK * 2);
        int kt0 = 0, nsteps = KT;
        if constexpr (PART) {
            kt0 = __builtin_amdgcn_readfirstlane((int)((long long)part * KT / nsplit));
            nsteps = __builtin_amdgcn_readfirstlane((int)((long long)(part + 1) * KT / nsplit) - kt0);
        }

        const __amdgpu_buffer_rsrc_t ra = GATHER ? make_rsrc(A, (uint32_t)(a_rows * K * 2))
                                                 : make_rsrc(A + (long long)tl.row0 * K, (uint32_t)rows * K * 2);
        const long long eoff = (long long)tl.e * K * N;
        const __amdgpu_buffer_rsrc_t rb0 = make_rsrc(B0 + eoff, (uint32_t)K * rowB);
        const __amdgpu_buffer_rsrc_t rb1 = make_rsrc((NMAT == 2 ? B1 : B0) + eoff, (uint32_t)K * rowB);

        f32x4_t acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // An expert held by one row tile has each of its weight slices read by one work
        // item only: those loads carry the non-temporal hint, so the one-pass weight
        // stream of the many short experts leaves L2 before the row tiles and weight
        // slices that the items of the long experts share.
        const bool wstream = tl.cnt == 1;
#define MOE_PP_ITEM(G_, AUX_) pp_item<G_, BM, NMAT, GATHER, AUX_>(lds, kt0, nsteps, nblk, tl, rows, n0, K, N, ra, rb0, \
                                                              rb1, gather_rows, wave, lane, a_rd, b_rd, g, wn, acc)
        if (grp == 0) {
            if (wstream) MOE_PP_ITEM(0, kWStream);
            else MOE_PP_ITEM(0, 0);
        } else {
            if (wstream) MOE_PP_ITEM(1, kWStream);
            else MOE_PP_ITEM(1, 0);
        }
#undef MOE_PP_ITEM
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the tail's zero loads land before LDS is reused
        __syncthreads();
        claim();                                            // the next work item, during the epilogue

        // a split item: store this part; only the last part to arrive goes on, adding the
        // parts in part order (the item's slots are consecutive in the part buffer)
        __amdgpu_buffer_rsrc_t rp;
        uint32_t wofs = 0;
        if constexpr (PART) {
            rp = make_rsrc(pbuf + (size_t)slot * nsplit * SLOT, (uint32_t)(nsplit * SLOT * 4));
            wofs = (uint32_t)((wave * FM * FN * 256 + lane * 4) * 4);
            if (nblk > 0) {
                const uint32_t pofs = (uint32_t)(part * SLOT * 4);
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        store_part(rp, pofs + wofs + (uint32_t)((fm * FN + fn) * 1024), acc[fm][fn]);
            }
            const SplitPart sp{nullptr, nullptr, part_cnt + slot, nsplit, SLOT};
            if (!split_arrive(sp, flag)) return;
        }
        if constexpr (PART)
            pp_write_split<BM, NMAT, ACT>(lds, rp, wofs, nsplit, nblk, row0, wn, l16, lq, tid, rows, n0, N,
                                          C + (long long)tl.row0 * N);
        else
            pp_write_out<BM, NMAT, ACT>(lds, [&](int fm, int fn) { return acc[fm][fn]; }, nblk, row0, wn, l16,
                                        lq, tid, rows, n0, N, C + (long long)tl.row0 * N);
    };

    // full rounds (every item when the launch does not split), then the split tail
    long long main_end;
    {
        const WorkSplit wsp(total, G, pbuf ? KT : 0);
        main_end = wsp.split == 1 ? total : wsp.full;
    }
    // Work order.  The static order gives workgroup b the work indices first, first + G, ...
    // (XCD b % 8 runs a contiguous chunk of G / 8 indices per round).  With item_q, XCD x's
    // workgroups instead take the indices the static order gives XCD x in order from a
    // counter (queue x), so the items running together on an XCD stay a contiguous window
    // of the order (the row tiles and weight slices they share stay shared) even when
    // items differ in length.  A workgroup whose queue is empty takes items from the next
    // XCD's queue, and so on round the eight, so no XCD idles while another has items
    // left (the queues' lengths differ with the launch's last round, and their items'
    // costs with the experts' tiles).  The claim for the next item is made during the
    // current one's epilogue; it reaches the other wavefronts through an LDS word, read
    // between two barriers (the word lies in the rings the next item's DMA fills).
    int* const fetch_word = flag + 1;
    // the work count: the items, or with the split the full rounds' items and the parts
    auto work_count = [&]() -> long long {
        const long long n = (long long)(*ntiles_p) * NT;
        return SPLIT ? WorkSplit(n, G, pbuf ? KT : 0).nwork : n;
    };
    // thread 0: the work index of claim c on this XCD's queue; past its end, an item of the
    // first other queue (in XCD order from this one) that still holds one, or -1.  A queue
    // once empty stays empty, so one pass that finds each queue empty (by its count or by
    // a claim past its end) proves all are.
    auto qlen_of = [&](int v) -> long long {
        const long long nw = work_count();
        const long long rounds = nw / G, rem = nw - rounds * G;
        return rounds * per_xcd + min(max(rem - (long long)v * per_xcd, 0LL), (long long)per_xcd);
    };
    // this XCD's queue length, fixed for the launch: the common case of resolve below is a
    // claim inside it, taken without reloading the tile count or 64-bit divisions (those had
    // made the hand-off between two items some 5k cycles)
    const int own_len = item_q ? __builtin_amdgcn_readfirstlane((int)qlen_of(xcd)) : 0;
    auto resolve = [&](int c) -> int {
        if (c < own_len) return (c / per_xcd) * G + xcd * per_xcd + c % per_xcd;
        const long long nw = work_count();
        const long long rounds = nw / G, rem = nw - rounds * G;
        auto qlen = [&](int v) {
            return rounds * per_xcd + min(max(rem - (long long)v * per_xcd, 0LL), (long long)per_xcd);
        };
        auto index = [&](int v, long long i) { return (int)((i / per_xcd) * G + (long long)v * per_xcd + i % per_xcd); };
        int seen[8];
#pragma unroll
        for (int i = 1; i < 8; ++i)
            seen[i] = __hip_atomic_load(item_q + ((xcd + i) & 7), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int i = 1; i < 8; ++i) {
            const int v = (xcd + i) & 7;
            const long long len = qlen(v);
            if (seen[i] >= len) continue;
            const int cv = atomicAdd(item_q + v, 1);
            if (cv < len) return index(v, cv);
        }
        return -1;
    };
    auto next = [&](long long cur) -> long long {
        if (!item_q) {
            const long long n = cur + G;
            return n < work_count() ? n : -1;
        }
        if (tid == 0) *fetch_word = resolve(cn);
        __syncthreads();
        const int v = *fetch_word;
        __syncthreads();
        return v;
    };
    long long w;
    if (item_q) {
        if (tid == 0) *fetch_word = resolve(atomicAdd(item_q + xcd, 1));
        __syncthreads();
        w = *fetch_word;
        __syncthreads();
    } else {
        w = first < work_count() ? first : -1;
    }
    // full items (every item when the launch does not split), then split parts; a queue
    // taken over from another XCD may hand out a full item after a part
    while (w >= 0) {
        for (; w >= 0 && w < main_end; w = next(w)) run_item(w, 0, 1, -1, std::false_type{});
        if constexpr (!SPLIT) break;                 // every index is below main_end
        else {
            // the split is derived again from the tile count (reloaded after the loop's
            // memory clobbers), so that none of it is held through the full items
            const WorkSplit wsp((long long)(*ntiles_p) * NT, G, pbuf ? KT : 0);
            for (; w >= main_end; w = next(w)) {
                long long item;
                int part, slot;
                wsp.item_of(w, item, part, slot);
                run_item(item, __builtin_amdgcn_readfirstlane(part), wsp.split,
                         __builtin_amdgcn_readfirstlane(slot), std::true_type{});
            }
        }
    }
}

// Grouped GEMM for BM-row tiles (256 or 320), ping-pong form (512 threads).  The two
// heights are launched together; whichever the tile builder chose runs, the other
// returns.  The SPLIT instance also splits the last round along K; the host launches it
// only where K allows a split, since the split's code alone slows the kernel's short-K
// items by about 2%.
template <int BM, int NMAT, int ACT, bool GATHER, bool SPLIT>
__global__ __launch_bounds__(512, 1) void k_grouped_gemm_pp(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ gather_rows,
    const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1, bf16_t* __restrict__ C,
    const Tile* __restrict__ tiles, const int32_t* __restrict__ ntiles_p, int K, int N,
    long long a_rows, float* __restrict__ part_buf, int* __restrict__ part_cnt, int* __restrict__ item_q) {
    extern __shared__ uint4 smem[];
    if (__builtin_amdgcn_readfirstlane(ntiles_p[1]) != BM) return;
    gemm_tiles_pp<BM, NMAT, ACT, GATHER, SPLIT>(smem, A, gather_rows, B0, B1, C, tiles, ntiles_p, K, N, a_rows,
                                                part_buf, part_cnt, item_q);
}

// ------------------------------------------------------------------------ tile list
// One workgroup of 256 threads (E <= 256).  Two candidate row-tile heights BMA and BMB
// (equal when the kernel has one shape): with wa / wb column blocks per row tile (both
// projections), the height giving fewer work items, sum_e ceil(count_e / BM) * w, wins
// (BMA on a tie).  Every item costs about the same K steps whatever its rows, so the
// item count is the cost.  Expert e then gets ceil(count_e / BM) tiles; ntiles[0] is the
// tile count and ntiles[1] the height chosen.
__global__ __launch_bounds__(256) void k_build_tiles(const int32_t* __restrict__ offsets, int E,
                                                     int BMA, int BMB, int wa, int wb,
                                                     Tile* __restrict__ tiles,
                                                     int32_t* __restrict__ ntiles, int* __restrict__ part_cnt) {
    // the grouped GEMMs' split-part counters start at zero (each launch leaves them so)
    static_assert(kPartSlots <= 256, "one counter per thread");
    if (part_cnt && threadIdx.x < kPartSlots) part_cnt[threadIdx.x] = 0;
    if (part_cnt && threadIdx.x < kGemmQueues) part_cnt[kPartSlots + threadIdx.x] = 0;   // the fetch counters
    __shared__ int buf[2][256];
    __shared__ long long cost[2][4];
    const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
    int r0 = 0, r1 = 0;
    if (e < E) {
        r0 = offsets[e];
        r1 = offsets[e + 1];
    }
    long long ca = (long long)((r1 - r0 + BMA - 1) / BMA) * wa;
    long long cb = (long long)((r1 - r0 + BMB - 1) / BMB) * wb;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        ca += __shfl_xor(ca, off);
        cb += __shfl_xor(cb, off);
    }
    if (lane == 0) {
        cost[0][wave] = ca;
        cost[1][wave] = cb;
    }
    __syncthreads();
    const long long ta = cost[0][0] + cost[0][1] + cost[0][2] + cost[0][3];
    const long long tb = cost[1][0] + cost[1][1] + cost[1][2] + cost[1][3];
    const int BM = tb < ta ? BMB : BMA;
    const int nt = (r1 - r0 + BM - 1) / BM;
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
    for (int i = 0; i < nt; ++i) tiles[base + i] = Tile{e, r0 + i * BM, min(r0 + (i + 1) * BM, r1), base, nt, 0, 0, 0};
    if (e == 255) {
        ntiles[0] = incl;
        ntiles[1] = BM;
    }
}

hipError_t launch_build_tiles(const int32_t* offsets, int E, int BMA, int BMB, int wa, int wb,
                              Tile* tiles, int32_t* ntiles, int* part_cnt, hipStream_t st) {
    hipLaunchKernelGGL(k_build_tiles, dim3(1), dim3(256), 0, st, offsets, E, BMA, BMB, wa, wb, tiles, ntiles,
                       part_cnt);
    return hipGetLastError();
}

void gemm_cfg_heights(GemmCfg c, int* bma, int* bmb) {
    switch (c) {
        case GEMM_M16: *bma = *bmb = 16; return;
        case GEMM_M64: *bma = *bmb = 64; return;
        case GEMM_M128: *bma = *bmb = 128; return;
        default: *bma = 256; *bmb = 320; return;     // chosen per launch by the tile builder
    }
}

// Column blocks of one row tile over both projections (first: N = F, second: N = H).
static int col_blocks(int BM, int H, int F, int swiglu) {
    int bn1, bn2;
    if (BM < 64) {
        bn1 = swiglu ? 128 : 256;
        bn2 = 256;
    } else if (BM == 320) {
        bn1 = swiglu ? LdsShape<320, 2>::BNm : LdsShape<320, 1>::BNm;
        bn2 = LdsShape<320, 1>::BNm;
    } else {
        bn1 = swiglu ? LdsShape<256, 2>::BNm : LdsShape<256, 1>::BNm;
        bn2 = LdsShape<256, 1>::BNm;
    }
    return (F + bn1 - 1) / bn1 + (H + bn2 - 1) / bn2;
}

hipError_t launch_build_tiles_for(const int32_t* offsets, int E, GemmCfg cfg, int H, int F, int swiglu,
                                  Tile* tiles, int32_t* ntiles, int* part_cnt, hipStream_t st) {
    int a, b;
    gemm_cfg_heights(cfg, &a, &b);
    return launch_build_tiles(offsets, E, a, b, col_blocks(a, H, F, swiglu), col_blocks(b, H, F, swiglu),
                              tiles, ntiles, part_cnt, st);
}

// ------------------------------------------------------------------------ launching
// Persistent grid: one workgroup per CU slot the kernel's LDS and registers allow,
// rounded to a multiple of 8 (the XCD count) and capped by the work-item bound.
template <typename KernT>
static hipError_t persistent_grid(KernT kern, size_t lds_bytes, bool& ready, int& occ_cache,
                                  long long max_items, unsigned& grid, int threads = 256) {
    if (!ready) {   // per process: properties of the code object
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)lds_bytes);
        if (e != hipSuccess) return e;
        int occ = 1;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, threads, lds_bytes) != hipSuccess || occ < 1)
            occ = 1;
        occ_cache = occ;
        ready = true;
    }
    long long G = (long long)device_cu_count() * occ_cache;
    const long long cap = ((max_items + 7) / 8) * 8;
    if (G > cap) G = cap;
    G = ((G + 7) / 8) * 8;
    if (G < 8) G = 8;
    grid = (unsigned)G;
    return hipSuccess;
}

// 320-row tiles of a launch pair in the ping-pong kernel (else the 4-wavefront kernel).
// Measured on the pages' worked shape (weights streamed from HBM), the ping-pong form
// with the same rings and row split matched the 4-wavefront kernel on the first
// projection and was 3% slower on the second, so the 4-wavefront kernel stays.
constexpr bool kPp320 = false;

// One ping-pong kernel of a launch pair (BM-row tiles), split-capable or not.
template <int BM, int NMAT, int ACT, bool GATHER, bool SPLIT>
static hipError_t run_pp(const void* A, long long a_rows, const int32_t* gather_rows, const void* B0,
                         const void* B1, void* C, const Tile* tiles, const int32_t* ntiles,
                         long long max_items, int K, int N, const SplitBuffers& sb, hipStream_t st) {
    static bool ready = false;
    static int occ = 1;
    unsigned G = 0;
    constexpr size_t pp_bytes = pp_lds_bytes<BM, NMAT>();
    auto kpp = k_grouped_gemm_pp<BM, NMAT, ACT, GATHER, SPLIT>;
    hipError_t e = persistent_grid(kpp, pp_bytes, ready, occ, max_items, G, 512);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kpp, dim3(G), dim3(512), pp_bytes, st, (const bf16_t*)A, gather_rows, (const bf16_t*)B0,
                       (const bf16_t*)B1, (bf16_t*)C, tiles, ntiles, K, N, a_rows, sb.parts, sb.counts,
                       G % 8 == 0 ? sb.queue : nullptr);
    return hipGetLastError();
}

template <int BM, int BMB, int NMAT, int WAVES_M, int ACT, bool GATHER>
static hipError_t run_gemm(const void* A, long long a_rows, const int32_t* gather_rows, const void* B0,
                           const void* B1, void* C, const Tile* tiles, const int32_t* ntiles,
                           long long max_items, int K, int N, const SplitBuffers& sb, hipStream_t st) {
    static bool ready = false;
    static int occ = 1;
    unsigned G = 0;
    if constexpr (BM < 64) {
        using S = GemmShape<BM, 256, NMAT, WAVES_M>;
        auto kern = k_grouped_gemm_bf16<BM, 256, NMAT, WAVES_M, ACT, GATHER>;
        hipError_t e = persistent_grid(kern, S::LDS_BYTES, ready, occ, max_items, G);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(G), dim3(256), S::LDS_BYTES, st, (const bf16_t*)A, gather_rows,
                           (const bf16_t*)B0, (const bf16_t*)B1, (bf16_t*)C, tiles, ntiles, K, N);
    } else {
        if constexpr (BM == 256 && BMB == 320) {
            // launch pair: 256-row tiles in the ping-pong kernel, 320-row tiles in the
            // 4-wavefront kernel; the one whose height was not chosen returns at once
            const bool split = !GATHER && sb.parts && (K + 31) / 32 >= 2 * kMinPartSteps;
            hipError_t e = split ? run_pp<256, NMAT, ACT, GATHER, !GATHER>(A, a_rows, gather_rows, B0, B1, C, tiles,
                                                                         ntiles, max_items, K, N, sb, st)
                                 : run_pp<256, NMAT, ACT, GATHER, false>(A, a_rows, gather_rows, B0, B1, C, tiles,
                                                                       ntiles, max_items, K, N, sb, st);
            if (e != hipSuccess) return e;
            if constexpr (kPp320) {
                return split ? run_pp<320, NMAT, ACT, GATHER, !GATHER>(A, a_rows, gather_rows, B0, B1, C, tiles,
                                                                       ntiles, max_items, K, N, sb, st)
                             : run_pp<320, NMAT, ACT, GATHER, false>(A, a_rows, gather_rows, B0, B1, C, tiles,
                                                                     ntiles, max_items, K, N, sb, st);
            }
            constexpr size_t lds_bytes = LdsShape<320, NMAT>::LDS_BYTES;
            auto kern = k_grouped_gemm_lds<320, 320, NMAT, ACT, GATHER>;
            e = persistent_grid(kern, lds_bytes, ready, occ, max_items, G);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(kern, dim3(G), dim3(256), lds_bytes, st, (const bf16_t*)A, gather_rows,
                               (const bf16_t*)B0, (const bf16_t*)B1, (bf16_t*)C, tiles, ntiles, K, N, a_rows,
                               sb.parts, sb.counts);
            return hipGetLastError();
        } else {
            constexpr size_t lds_bytes = LdsPair<BM, BMB>::template bytes<NMAT>();
            auto kern = k_grouped_gemm_lds<BM, BMB, NMAT, ACT, GATHER>;
            hipError_t e = persistent_grid(kern, lds_bytes, ready, occ, max_items, G);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(kern, dim3(G), dim3(256), lds_bytes, st, (const bf16_t*)A, gather_rows,
                               (const bf16_t*)B0, (const bf16_t*)B1, (bf16_t*)C, tiles, ntiles, K, N, a_rows,
                               sb.parts, sb.counts);
        }
    }
    return hipGetLastError();
}

template <int BM, int BMB, int WAVES_M>
static hipError_t run_ffn(const void* a, long long a_rows, const int32_t* gather_rows, const void* w_in,
                          const void* w_up, const void* w_out, void* h, void* y,
                          const Tile* tiles, const int32_t* ntiles, long long max_tiles,
                          int H, int F, int swiglu, const SplitBuffers& sb, const hipEvent_t* ev, hipStream_t st) {
    hipError_t e;
    if (ev && (e = hipEventRecord(ev[0], st)) != hipSuccess) return e;
    // work items (row tiles x column blocks) bound the persistent grid: the larger of the
    // two shapes' counts (max_tiles is counted for the lower height)
    const long long items = max_tiles * std::max(col_blocks(BM, H, F, swiglu), col_blocks(BMB, H, F, swiglu));
    if (swiglu) {
        e = gather_rows ? run_gemm<BM, BMB, 2, WAVES_M, 1, true>(a, a_rows, gather_rows, w_in, w_up, h, tiles, ntiles, items, H, F, sb, st)
                        : run_gemm<BM, BMB, 2, WAVES_M, 1, false>(a, a_rows, nullptr, w_in, w_up, h, tiles, ntiles, items, H, F, sb, st);
    } else {
        e = gather_rows ? run_gemm<BM, BMB, 1, WAVES_M, 1, true>(a, a_rows, gather_rows, w_in, nullptr, h, tiles, ntiles, items, H, F, sb, st)
                        : run_gemm<BM, BMB, 1, WAVES_M, 1, false>(a, a_rows, nullptr, w_in, nullptr, h, tiles, ntiles, items, H, F, sb, st);
    }
    if (e != hipSuccess) return e;
    if (ev && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
    SplitBuffers sb2 = sb;             // the second projection's own fetch counters
    if (sb2.queue) sb2.queue += 8;
    e = run_gemm<BM, BMB, 1, WAVES_M, 0, false>(h, 0, nullptr, w_out, nullptr, y, tiles, ntiles, items, F, H, sb2, st);
    if (e == hipSuccess && ev) e = hipEventRecord(ev[2], st);
    return e;
}

hipError_t launch_grouped_ffn_bf16(const void* a, long long a_rows, const int32_t* gather_rows,
                                   const void* w_in, const void* w_up, const void* w_out,
                                   void* h, void* y, const Tile* tiles, const int32_t* ntiles,
                                   long long max_tiles, GemmCfg cfg, int H, int F, int swiglu,
                                   const SplitBuffers& sb, const hipEvent_t* ev, hipStream_t st) {
    switch (cfg) {
        case GEMM_M16:
            return run_ffn<16, 16, 1>(a, a_rows, gather_rows, w_in, w_up, w_out, h, y, tiles, ntiles, max_tiles, H, F, swiglu, sb, ev, st);
        case GEMM_M64:
            return run_ffn<64, 64, 2>(a, a_rows, gather_rows, w_in, w_up, w_out, h, y, tiles, ntiles, max_tiles, H, F, swiglu, sb, ev, st);
        case GEMM_M128:
            return run_ffn<128, 128, 2>(a, a_rows, gather_rows, w_in, w_up, w_out, h, y, tiles, ntiles, max_tiles, H, F, swiglu, sb, ev, st);
        default:
            return run_ffn<256, 320, 2>(a, a_rows, gather_rows, w_in, w_up, w_out, h, y, tiles, ntiles, max_tiles, H, F, swiglu, sb, ev, st);
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
                                  const hipEvent_t* ev, hipStream_t st) {
    const dim3 blk(256);
    hipError_t e;
    if (ev && (e = hipEventRecord(ev[0], st)) != hipSuccess) return e;
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
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
    const dim3 g2((unsigned)max_tiles, (unsigned)((H + 63) / 64));
    hipLaunchKernelGGL((k_grouped_gemm_f32<1, 0, false>), g2, blk, 0, st, (const float*)h, nullptr, (const float*)w_out, nullptr, (float*)y, tiles, ntiles, F, H);
    e = hipGetLastError();
    if (e == hipSuccess && ev) e = hipEventRecord(ev[2], st);
    return e;
}

}  // namespace moe
