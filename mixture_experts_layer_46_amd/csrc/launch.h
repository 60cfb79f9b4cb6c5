// Host-side launchers of the MoE kernels (one per kernel family).  Each enqueues on
// `st` and returns the launch status; shapes were validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Sets the calling thread's moe_last_error() text and returns st (for entry points
// defined outside api.hip).
moe_status report_error(moe_status st, const char* text);

// pairs per segment of the grouping kernels (one wavefront handles one segment)
constexpr int kSeg = 512;

// One grouped-GEMM row tile: rows [row0, row1) of expert `e` (row1 - row0 <= BM).  The
// list is expert-major; `first` is the index of expert e's first tile and `cnt` its
// number of tiles, so a work item can find its expert's tiles in O(1).
struct Tile {
    int e, row0, row1, first, cnt, pad0, pad1, pad2;
};

// Workspace of the bf16 grouped GEMM's split of the last round (see grouped_gemm.hip):
// kGemmPartSlots slots of up to kGemmPartSlotFloats fp32 accumulators, and as many int
// counters (zeroed by the tile builder).  NULL buffers switch the split off.
constexpr int kGemmPartSlots = 256;
constexpr size_t kGemmPartSlotFloats = 256 * 256;    // the largest tile, BM x BN
// Per-XCD work-item counters of the ping-pong GEMM's ordered fetch: 8 for the first
// projection, 8 for the second, right after the part counters (and zeroed with them).
constexpr int kGemmQueues = 16;
struct SplitBuffers {
    float* parts;
    int* counts;
    int* queue;       // this launch's 8 per-XCD counters (NULL: static order)
};

// Tile configurations of the bf16 grouped GEMM.  GEMM_M256 lets the tile builder choose
// 256- or 320-row tiles per launch from the actual per-expert counts.
enum GemmCfg { GEMM_M16 = 0, GEMM_M64 = 1, GEMM_M128 = 2, GEMM_M256 = 3 };
// the row-tile heights a configuration may use (*bma == *bmb: one shape)
void gemm_cfg_heights(GemmCfg c, int* bma, int* bmb);

// K splits of the gate projection (partial sums [splits][T][E]) for a layer shape
int gate_splits(long long T, int H, int E, int dtype);   // split-K ranges of the gate projection
// whether the bf16 gate splits W_g into bf16 planes once per call (planes: 3 * E *
// gate_plane_k(H) bf16 of workspace, K-step-major); `planes` NULL keeps the split inside
// each workgroup (moe_route, which has no workspace)
bool gate_uses_planes(long long T, int dtype);
__host__ __device__ inline int gate_plane_k(int H) { return (H + 31) / 32 * 32; }   // H in whole K steps
hipError_t launch_gate_logits(const void* x, int dtype, const float* wg, float* out,
                              long long T, int H, int E, int splits, bf16_t* planes, hipStream_t st);
// top-k over the sum of `nparts` partial logits; the sum goes to logits_out if not NULL
hipError_t launch_topk(const float* logits, int nparts, float* logits_out, const float* bias,
                       int32_t* idx, float* w, long long T, int E, int k, unsigned flags,
                       hipStream_t st);

hipError_t launch_group(const int32_t* topk_idx, long long P, int k, int E, int capacity,
                        int32_t* segcnt, int32_t* counts, int32_t* offsets,
                        int32_t* sorted_token, int32_t* row_of_pair, hipStream_t st);
hipError_t launch_gather(const void* x, const int32_t* sorted_token, const int32_t* offsets,
                         int E, void* x_perm, long long P, int H, int esize, hipStream_t st);

// tile list for heights BMA / BMB (the one with fewer work items; wa, wb = column blocks
// per row tile); ntiles[0] = tile count, ntiles[1] = the height chosen
hipError_t launch_build_tiles(const int32_t* offsets, int E, int BMA, int BMB, int wa, int wb,
                              Tile* tiles, int32_t* ntiles, int* part_cnt, hipStream_t st);
// the same for a bf16 configuration of the grouped FFN
hipError_t launch_build_tiles_for(const int32_t* offsets, int E, GemmCfg cfg, int H, int F, int swiglu,
                                  Tile* tiles, int32_t* ntiles, int* part_cnt, hipStream_t st);

// grouped FFN.  A rows: x_perm rows directly (gather_rows == NULL) or x[gather_rows[r]]
// with x holding a_rows rows (its bytes must stay below 2^32 for the 32-bit buffer
// offsets of the row-tile kernels).  ev: NULL, or three events recorded on `st` before
// the first projection, between the two projections and after the second.
hipError_t launch_grouped_ffn_bf16(const void* a, long long a_rows, const int32_t* gather_rows,
                                   const void* w_in, const void* w_up, const void* w_out,
                                   void* h, void* y, const Tile* tiles, const int32_t* ntiles,
                                   long long max_tiles, GemmCfg cfg, int H, int F, int swiglu,
                                   const SplitBuffers& sb, const hipEvent_t* ev, hipStream_t st);
hipError_t launch_grouped_ffn_f32(const void* a, const int32_t* gather_rows,
                                  const void* w_in, const void* w_up, const void* w_out,
                                  void* h, void* y, const Tile* tiles, const int32_t* ntiles,
                                  long long max_tiles, int H, int F, int swiglu,
                                  const hipEvent_t* ev, hipStream_t st);

hipError_t launch_combine(const void* y_perm, const int32_t* row_of_pair, const float* w,
                          void* out, long long T, int k, int H, int dtype, hipStream_t st);

hipError_t launch_router_stats(const float* logits, const float* bias, const int32_t* counts,
                               const int32_t* offsets, float* stats, long long T, int E, int k,
                               int capacity, hipStream_t st);

int device_cu_count();

}  // namespace moe
