// Grouping of token-expert pairs by expert: histogram, prefix sum, stable permutation
// and row gather.
//
// Pages cited (by title and section):
//   [FourStage]  "MoE显存与计算开销四阶段手算指南" (bjdmk.com.cn/news/5154310)
//   [Principles] "MoE混合专家模型计算原理与推理部署实战解析" (sheratonhq.com/news/207562)
//
// [Principles §5.1] steps 2-3: count the pairs of each expert, prefix-sum the counts
// into buffer offsets, and move every pair to a contiguous expert-major buffer
// ([FourStage §2.3]: the rows of expert i form one [N_i, H] block; [FourStage §4.3]:
// the block must be contiguous).  The permutation is a stable counting sort on the
// pair index p = t*k + j, so within an expert rows follow token order and the result
// is independent of scheduling (no global atomics):
//   1. k_seg_count   one wavefront per 512-pair segment: per-expert counts of the
//                    segment (LDS atomics, whose sum is order-free)
//   2. k_seg_scan    one workgroup: per expert, exclusive prefix over segments (the
//                    rank base of each segment), totals, capacity cut, offsets
//   3. k_seg_scatter one wavefront per segment: the rank of each pair among equal
//                    experts of its 64-pair round comes from a match mask built with
//                    ballots over the index bits plus a popcount of lower lanes
#include "common.h"
#include "launch.h"

namespace moe {

__global__ __launch_bounds__(256) void k_seg_count(const int32_t* __restrict__ idx,
                                                   long long P, int E, long long NS,
                                                   int32_t* __restrict__ segcnt) {
    __shared__ int32_t hist[4][256];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int e = lane; e < 256; e += 64) hist[w][e] = 0;
    __syncthreads();
    const long long s = (long long)blockIdx.x * 4 + w;
    if (s < NS) {
        for (int r = 0; r < kSeg / 64; ++r) {
            const long long p = s * kSeg + r * 64 + lane;
            if (p < P) {
                const unsigned e = (unsigned)idx[p];
                if (e < (unsigned)E) atomicAdd(&hist[w][e], 1);   // out-of-range ids are dropped
            }
        }
    }
    __syncthreads();
    if (s < NS)
        for (int e = lane; e < E; e += 64) segcnt[s * E + e] = hist[w][e];
}

// One workgroup of 256 threads (E <= 256).  segcnt[s][e] is replaced by the number of
// pairs of expert e in segments before s (the rank base of segment s).
__global__ __launch_bounds__(256) void k_seg_scan(int32_t* __restrict__ segcnt, long long NS,
                                                  int E, int capacity,
                                                  int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ offsets) {
    __shared__ int32_t buf[2][256];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        // segments in batches of 16: the batch's loads are issued together, so the chain
        // of dependent loads and stores no longer costs one memory latency per segment
        constexpr int B = 16;
        for (long long s0 = 0; s0 < NS; s0 += B) {
            int c[B];
#pragma unroll
            for (int j = 0; j < B; ++j) c[j] = s0 + j < NS ? segcnt[(s0 + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < B; ++j) {
                if (s0 + j < NS) segcnt[(s0 + j) * E + e] = run;
                run += c[j];
            }
        }
        counts[e] = run;
    }
    const int kept = (e < E) ? (capacity > 0 ? min(run, capacity) : run) : 0;
    // inclusive scan over the 256 experts (Hillis-Steele, double buffered)
    int cur = 0;
    buf[0][e] = kept;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const int v = buf[cur][e] + (e >= off ? buf[cur][e - off] : 0);
        buf[cur ^ 1][e] = v;
        cur ^= 1;
        __syncthreads();
    }
    const int incl = buf[cur][e];
    if (e < E) offsets[e] = incl - kept;
    if (e == E - 1) offsets[E] = incl;
}

__global__ __launch_bounds__(256) void k_seg_scatter(const int32_t* __restrict__ idx, long long P,
                                                     int k, int E, int nbits, int capacity,
                                                     long long NS,
                                                     const int32_t* __restrict__ segbase,
                                                     const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ sorted_token,
                                                     int32_t* __restrict__ row_of_pair) {
    __shared__ int32_t run[4][256];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int e = lane; e < 256; e += 64) run[w][e] = 0;
    __syncthreads();
    const long long s = (long long)blockIdx.x * 4 + w;
    if (s >= NS) return;
    const uint64_t lt = lanemask_lt();
    // the segment's expert ids, then their rank bases and offsets, all loaded before the
    // ranking, so the segment costs two memory latencies instead of two per round
    constexpr int R = kSeg / 64;
    int ev[R], base[R], off[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const long long p = s * kSeg + r * 64 + lane;
        ev[r] = p < P ? idx[p] : -1;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool valid = (unsigned)ev[r] < (unsigned)E;
        base[r] = valid ? segbase[s * E + ev[r]] : 0;
        off[r] = valid ? offsets[ev[r]] : 0;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const long long p = s * kSeg + r * 64 + lane;
        const bool inside = p < P;
        const bool valid = inside && (unsigned)ev[r] < (unsigned)E;
        const int e = valid ? ev[r] : 0;
        // lanes of this round holding the same expert id
        uint64_t same = ballot64(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t m = ballot64(valid && bit);
            same &= bit ? m : ~m;
        }
        const int before = __popcll(same & lt);
        int row = -1;
        if (valid) {
            const int rank = base[r] + run[w][e] + before;
            if (capacity <= 0 || rank < capacity) row = off[r] + rank;
        }
        __builtin_amdgcn_wave_barrier();
        if (valid && before == 0) run[w][e] += __popcll(same);   // one leader per expert
        __builtin_amdgcn_wave_barrier();
        if (inside) {
            row_of_pair[p] = row;
            if (row >= 0) sorted_token[row] = (int32_t)(p / k);
        }
    }
}

// x_perm[r] = x[sorted_token[r]] for r < offsets[E]; one workgroup per grouped row,
// 16-byte loads and stores.
__global__ __launch_bounds__(256) void k_gather_rows(const uint4* __restrict__ x,
                                                     const int32_t* __restrict__ sorted_token,
                                                     const int32_t* __restrict__ offsets, int E,
                                                     uint4* __restrict__ x_perm, int chunks) {
    const long long r = blockIdx.x;
    if (r >= offsets[E]) return;
    const long long src = (long long)sorted_token[r] * chunks;
    const long long dst = r * chunks;
    for (int c = threadIdx.x; c < chunks; c += 256) x_perm[dst + c] = x[src + c];
}

hipError_t launch_group(const int32_t* topk_idx, long long P, int k, int E, int capacity,
                        int32_t* segcnt, int32_t* counts, int32_t* offsets,
                        int32_t* sorted_token, int32_t* row_of_pair, hipStream_t st) {
    const long long NS = (P + kSeg - 1) / kSeg;
    const unsigned nblk = (unsigned)((NS + 3) / 4);
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    hipLaunchKernelGGL(k_seg_count, dim3(nblk), dim3(256), 0, st, topk_idx, P, E, NS, segcnt);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_seg_scan, dim3(1), dim3(256), 0, st, segcnt, NS, E, capacity, counts,
                       offsets);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_seg_scatter, dim3(nblk), dim3(256), 0, st, topk_idx, P, k, E, nbits,
                       capacity, NS, segcnt, offsets, sorted_token, row_of_pair);
    return hipGetLastError();
}

hipError_t launch_gather(const void* x, const int32_t* sorted_token, const int32_t* offsets,
                         int E, void* x_perm, long long P, int H, int esize, hipStream_t st) {
    const int chunks = H * esize / 16;
    hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)P), dim3(256), 0, st, (const uint4*)x,
                       sorted_token, offsets, E, (uint4*)x_perm, chunks);
    return hipGetLastError();
}

}  // namespace moe
