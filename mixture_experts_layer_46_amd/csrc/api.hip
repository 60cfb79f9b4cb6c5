// C ABI of the MoE layer forward: argument checks, workspace carve-up, launches.
// Declarations, argument meaning, layouts, ownership and error behaviour: include/moe.h.
#include <algorithm>
#include <cmath>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "common.h"
#include "launch.h"
#include "moe.h"

namespace moe {

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

moe_status hip_fail(hipError_t e, const char* where) {
    return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

// Workspace layout shared by every entry point (offsets from the workspace base).
struct Layout {
    size_t logits, planes, topk_idx, topk_w, counts, offsets, segcnt, sorted_token, row_of_pair,
        tiles, ntiles, part_cnt, parts, h, y, total;
};

long long max_tiles_for(long long P, int E, int BM) {
    return (P + BM - 1) / BM + (P < E ? P : E);
}

// Row-tile height of the grouped GEMM from the mean rows per expert (host only knows
// T*k/E; per-expert counts stay on the device).
GemmCfg pick_cfg(const moe_shape& s) {
    const double mean = (double)s.T * s.k / s.E;
    if (mean <= 24) return GEMM_M16;
    if (mean <= 80) return GEMM_M64;
    if (mean <= 160) return GEMM_M128;
    return GEMM_M256;                    // 256 or 320 rows, chosen on the device
}

Layout layout_of(const moe_shape& s) {
    const size_t es = s.dtype == MOE_F32 ? 4 : 2;
    const size_t P = (size_t)s.T * s.k;
    const size_t NS = (P + kSeg - 1) / kSeg;
    Layout L{};
    size_t o = 0;
    L.logits = o;       o += up((size_t)gate_splits(s.T, s.H, s.E, s.dtype) * s.T * s.E * 4);
    L.planes = o;       o += gate_uses_planes(s.T, s.dtype) ? up((size_t)3 * s.E * gate_plane_k(s.H) * 2) : 0;
    L.topk_idx = o;     o += up(P * 4);
    L.topk_w = o;       o += up(P * 4);
    L.counts = o;       o += up((size_t)s.E * 4);
    L.offsets = o;      o += up((size_t)(s.E + 1) * 4);
    L.segcnt = o;       o += up(NS * s.E * 4);
    L.sorted_token = o; o += up(P * 4);
    L.row_of_pair = o;  o += up(P * 4);
    L.tiles = o;        o += up((size_t)max_tiles_for((long long)P, s.E, 16) * sizeof(Tile));
    L.ntiles = o;       o += up(4);
    // the bf16 grouped GEMM's split of the last round: part slots and their counters
    const bool split = s.dtype == MOE_BF16 && pick_cfg(s) != GEMM_M16;
    L.part_cnt = o;     o += split ? up((size_t)(kGemmPartSlots + kGemmQueues) * 4) : 0;
    L.parts = o;        o += split ? up((size_t)kGemmPartSlots * kGemmPartSlotFloats * 4) : 0;
    L.h = o;            o += up(P * s.F * es);
    L.y = o;            o += up(P * s.H * es);
    L.total = o;
    return L;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

moe_status check_shape(const moe_shape* s) {
    if (!s) return fail(MOE_ERR_NULL, "shape is NULL");
    if (s->T < 0) return fail(MOE_ERR_SHAPE, "T = %lld < 0", (long long)s->T);
    if (s->H <= 0 || s->E <= 0 || s->F <= 0 || s->k <= 0)
        return fail(MOE_ERR_SHAPE, "H, E, F, k must be positive (H=%d E=%d F=%d k=%d)", s->H, s->E, s->F, s->k);
    if (s->k > s->E) return fail(MOE_ERR_SHAPE, "k = %d > E = %d", s->k, s->E);
    if (s->E > 256) return fail(MOE_ERR_UNSUPPORTED, "E = %d > 256 is not supported", s->E);
    if (s->k > 8) return fail(MOE_ERR_UNSUPPORTED, "k = %d > 8 is not supported", s->k);
    if (s->H % 8 || s->F % 8) return fail(MOE_ERR_UNSUPPORTED, "H and F must be multiples of 8 (H=%d F=%d)", s->H, s->F);
    if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "dtype %d unknown", s->dtype);
    if (s->ffn != MOE_FFN_SILU2 && s->ffn != MOE_FFN_SWIGLU) return fail(MOE_ERR_UNSUPPORTED, "ffn %d unknown", s->ffn);
    if (s->flags & ~(MOE_FLAG_BIAS_SELECT_ONLY | MOE_FLAG_NO_RENORM))
        return fail(MOE_ERR_UNSUPPORTED, "unknown flag bits 0x%x", s->flags);
    if (s->capacity < 0) return fail(MOE_ERR_SHAPE, "capacity = %d < 0", s->capacity);
    const long long P = s->T * (long long)s->k;
    if (s->T >= (1ll << 31) || P >= (1ll << 31)) return fail(MOE_ERR_SHAPE, "T*k = %lld >= 2^31", P);
    const long long mx = s->H > s->F ? s->H : s->F;
    if ((double)P * (double)mx >= 4.0e18) return fail(MOE_ERR_SHAPE, "T*k*max(H,F) too large");
    // the grouped GEMM reads one expert matrix (plus up to 128 rows past its end) and the
    // token matrix x through buffer resources with 32-bit byte offsets, and marks a chunk
    // it must not load with the offset 2^31, which reads zeros only while the buffer is
    // shorter than that
    const long long es = s->dtype == MOE_F32 ? 4 : 2;
    if (((long long)s->H + 128) * s->F * es >= (1ll << 31) || ((long long)s->F + 128) * s->H * es >= (1ll << 31))
        return fail(MOE_ERR_UNSUPPORTED, "one expert matrix (H=%d x F=%d, plus 128 rows) must stay below 2 GiB",
                    s->H, s->F);
    if (s->T * (long long)s->H * es >= (1ll << 31))
        return fail(MOE_ERR_UNSUPPORTED, "x (T=%lld x H=%d) must stay below 2 GiB", (long long)s->T, s->H);
    // the bf16 gate's weight planes are read the same way
    if (gate_uses_planes(s->T, s->dtype) && 3ll * s->E * gate_plane_k(s->H) * 2 >= (1ll << 31))
        return fail(MOE_ERR_UNSUPPORTED, "the gate's weight planes (3 x E=%d x H=%d bf16) must stay below 2 GiB",
                    s->E, s->H);
    return MOE_OK;
}

#define REQ(p, name)                                                     \
    do {                                                                 \
        if (!(p)) return fail(MOE_ERR_NULL, "%s is NULL", name);         \
        if (!aligned16(p)) return fail(MOE_ERR_ALIGN, "%s is not 16-byte aligned", name); \
    } while (0)
#define OPT(p, name)                                                     \
    do {                                                                 \
        if ((p) && !aligned16(p)) return fail(MOE_ERR_ALIGN, "%s is not 16-byte aligned", name); \
    } while (0)
#define HIPCHK(expr, where)                                              \
    do {                                                                 \
        hipError_t e_ = (expr);                                          \
        if (e_ != hipSuccess) return hip_fail(e_, where);                \
    } while (0)

moe_status check_ws(const moe_shape& s, const void* ws, size_t ws_bytes) {
    const size_t need = layout_of(s).total;
    if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (!aligned16(ws)) return fail(MOE_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, need);
    return MOE_OK;
}


// Shape and pointer checks of the whole-layer entry points.
moe_status check_forward_args(const moe_shape* shape, const void* x, const float* w_gate, const float* bias,
                              const void* w_in, const void* w_up, const void* w_out, const void* out) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    REQ(x, "x");
    REQ(w_gate, "w_gate");
    OPT(bias, "bias");
    REQ(w_in, "w_in");
    REQ(w_out, "w_out");
    REQ(out, "out");
    if (shape->ffn == MOE_FFN_SWIGLU) REQ(w_up, "w_up");
    else if (w_up) return fail(MOE_ERR_SHAPE, "w_up must be NULL for the SiLU two-layer FFN");
    return MOE_OK;
}

moe_status run_grouped(const moe_shape& s, const void* a, const int32_t* gather_rows,
                       const int32_t* offsets, const void* w_in, const void* w_up,
                       const void* w_out, void* y, void* ws, const hipEvent_t* ev,
                       hipStream_t st) {
    const Layout L = layout_of(s);
    const long long P = s.T * (long long)s.k;
    const int swiglu = s.ffn == MOE_FFN_SWIGLU;
    Tile* tiles = at<Tile>(ws, L.tiles);
    int32_t* ntiles = at<int32_t>(ws, L.ntiles);
    if (s.dtype == MOE_F32) {
        const int BM = 64;
        HIPCHK(launch_build_tiles(offsets, s.E, BM, BM, 1, 1, tiles, ntiles, nullptr, st), "build_tiles");
        HIPCHK(launch_grouped_ffn_f32(a, gather_rows, w_in, w_up, w_out, at<void>(ws, L.h), y, tiles,
                                      ntiles, max_tiles_for(P, s.E, BM), s.H, s.F, swiglu, ev, st),
               "grouped_ffn_f32");
        return MOE_OK;
    }
    const GemmCfg cfg = pick_cfg(s);
    int bma, bmb;
    gemm_cfg_heights(cfg, &bma, &bmb);
    SplitBuffers sb{nullptr, nullptr, nullptr};
    if (cfg != GEMM_M16)
        sb = SplitBuffers{at<float>(ws, L.parts), at<int>(ws, L.part_cnt), at<int>(ws, L.part_cnt) + kGemmPartSlots};
    HIPCHK(launch_build_tiles_for(offsets, s.E, cfg, s.H, s.F, swiglu, tiles, ntiles, sb.counts, st), "build_tiles");
    HIPCHK(launch_grouped_ffn_bf16(a, gather_rows ? s.T : 0, gather_rows, w_in, w_up, w_out, at<void>(ws, L.h), y, tiles,
                                   ntiles, max_tiles_for(P, s.E, std::min(bma, bmb)), cfg, s.H, s.F, swiglu, sb, ev, st),
           "grouped_ffn_bf16");
    return MOE_OK;
}

// Scratch of moe_forward_noalloc: a file-scope device array (each GPU the library runs on
// holds its own copy until the process ends).  Host code never uses the array's name as
// an address (on the host it is only a stand-in): it uses the device address that
// hipGetSymbolAddress returns, looked up once per device.
constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on the first call on that device).
moe_status scratch_of_current_device(void** out) {
    int dev = -1;
    HIPCHK(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

moe_status report_error(moe_status st, const char* text) { return fail(st, "%s", text); }

int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_workspace_size(const moe_shape* shape, size_t* bytes) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (!bytes) return fail(MOE_ERR_NULL, "bytes is NULL");
    *bytes = layout_of(*shape).total;
    return MOE_OK;
}

moe_status moe_route(const moe_shape* shape, const void* x, const float* w_gate, const float* bias,
                     float* logits, int32_t* topk_idx, float* topk_w, hipStream_t stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape& s = *shape;
    if (x) {
        OPT(x, "x");
        REQ(w_gate, "w_gate");
        REQ(logits, "logits");
    } else {
        REQ(logits, "logits (input when x is NULL)");
    }
    OPT(bias, "bias");
    REQ(topk_idx, "topk_idx");
    REQ(topk_w, "topk_w");
    if (s.T == 0) return MOE_OK;
    (void)hipGetLastError();
    if (x) HIPCHK(launch_gate_logits(x, s.dtype, w_gate, logits, s.T, s.H, s.E, 1, nullptr, stream), "gate_logits");
    HIPCHK(launch_topk(logits, 1, nullptr, bias, topk_idx, topk_w, s.T, s.E, s.k, s.flags, stream), "topk");
    return MOE_OK;
}

moe_status moe_permute(const moe_shape* shape, const int32_t* topk_idx, const void* x,
                       int32_t* counts, int32_t* offsets, int32_t* sorted_token,
                       int32_t* row_of_pair, void* x_perm, void* workspace, size_t ws_bytes,
                       hipStream_t stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape& s = *shape;
    REQ(topk_idx, "topk_idx");
    REQ(counts, "counts");
    REQ(offsets, "offsets");
    REQ(sorted_token, "sorted_token");
    REQ(row_of_pair, "row_of_pair");
    OPT(x, "x");
    OPT(x_perm, "x_perm");
    if ((x == nullptr) != (x_perm == nullptr)) return fail(MOE_ERR_NULL, "x and x_perm must be given together");
    if ((st = check_ws(s, workspace, ws_bytes)) != MOE_OK) return st;
    if (s.T == 0) return MOE_OK;
    (void)hipGetLastError();
    const Layout L = layout_of(s);
    const long long P = s.T * (long long)s.k;
    HIPCHK(launch_group(topk_idx, P, s.k, s.E, s.capacity, at<int32_t>(workspace, L.segcnt), counts,
                        offsets, sorted_token, row_of_pair, stream),
           "group");
    if (x)
        HIPCHK(launch_gather(x, sorted_token, offsets, s.E, x_perm, P, s.H, s.dtype == MOE_F32 ? 4 : 2, stream),
               "gather");
    return MOE_OK;
}

moe_status moe_grouped_ffn(const moe_shape* shape, const void* x_perm, const int32_t* offsets,
                           const void* w_in, const void* w_up, const void* w_out, void* y_perm,
                           void* workspace, size_t ws_bytes, hipStream_t stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape& s = *shape;
    REQ(x_perm, "x_perm");
    REQ(offsets, "offsets");
    REQ(w_in, "w_in");
    REQ(w_out, "w_out");
    REQ(y_perm, "y_perm");
    if (s.ffn == MOE_FFN_SWIGLU) REQ(w_up, "w_up");
    else if (w_up) return fail(MOE_ERR_SHAPE, "w_up must be NULL for the SiLU two-layer FFN");
    if ((st = check_ws(s, workspace, ws_bytes)) != MOE_OK) return st;
    if (s.T == 0) return MOE_OK;
    (void)hipGetLastError();
    return run_grouped(s, x_perm, nullptr, offsets, w_in, w_up, w_out, y_perm, workspace, nullptr, stream);
}

moe_status moe_combine(const moe_shape* shape, const void* y_perm, const int32_t* row_of_pair,
                       const float* topk_w, void* out, hipStream_t stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape& s = *shape;
    REQ(y_perm, "y_perm");
    REQ(row_of_pair, "row_of_pair");
    REQ(topk_w, "topk_w");
    REQ(out, "out");
    if (s.T == 0) return MOE_OK;
    (void)hipGetLastError();
    HIPCHK(launch_combine(y_perm, row_of_pair, topk_w, out, s.T, s.k, s.H, s.dtype, stream), "combine");
    return MOE_OK;
}

moe_status moe_forward_timed(const moe_shape* shape, const void* x, const float* w_gate, const float* bias,
                             const void* w_in, const void* w_up, const void* w_out, void* out,
                             void* workspace, size_t ws_bytes, const hipEvent_t* events, hipStream_t stream) {
    moe_status st = check_forward_args(shape, x, w_gate, bias, w_in, w_up, w_out, out);
    if (st != MOE_OK) return st;
    const moe_shape& s = *shape;
    if ((st = check_ws(s, workspace, ws_bytes)) != MOE_OK) return st;
    if (events)
        for (int i = 0; i < MOE_STAGE_EVENTS; ++i)
            if (events[i] == nullptr) return fail(MOE_ERR_NULL, "events[%d] is NULL", i);
    if (s.T == 0) return MOE_OK;
    (void)hipGetLastError();
    const Layout L = layout_of(s);
    const long long P = s.T * (long long)s.k;
    float* logits = at<float>(workspace, L.logits);
    int32_t* idx = at<int32_t>(workspace, L.topk_idx);
    float* gw = at<float>(workspace, L.topk_w);
    int32_t* offsets = at<int32_t>(workspace, L.offsets);
    int32_t* sorted_token = at<int32_t>(workspace, L.sorted_token);
    int32_t* row_of_pair = at<int32_t>(workspace, L.row_of_pair);
    const int splits = gate_splits(s.T, s.H, s.E, s.dtype);
    if (events) HIPCHK(hipEventRecord(events[0], stream), "stage event");
    bf16_t* planes = gate_uses_planes(s.T, s.dtype) ? at<bf16_t>(workspace, L.planes) : nullptr;
    HIPCHK(launch_gate_logits(x, s.dtype, w_gate, logits, s.T, s.H, s.E, splits, planes, stream), "gate_logits");
    HIPCHK(launch_topk(logits, splits, nullptr, bias, idx, gw, s.T, s.E, s.k, s.flags, stream), "topk");
    if (events) HIPCHK(hipEventRecord(events[1], stream), "stage event");
    HIPCHK(launch_group(idx, P, s.k, s.E, s.capacity, at<int32_t>(workspace, L.segcnt),
                        at<int32_t>(workspace, L.counts), offsets, sorted_token, row_of_pair, stream),
           "group");
    // the first projection reads x rows through sorted_token: no x_perm copy.  Stage
    // events 2..4 are recorded by the grouped FFN (before, between and after its two
    // projections; the tile list is built before event 2).
    st = run_grouped(s, x, sorted_token, offsets, w_in, w_up, w_out, at<void>(workspace, L.y),
                     workspace, events ? events + 2 : nullptr, stream);
    if (st != MOE_OK) return st;
    HIPCHK(launch_combine(at<void>(workspace, L.y), row_of_pair, gw, out, s.T, s.k, s.H, s.dtype, stream),
           "combine");
    if (events) HIPCHK(hipEventRecord(events[5], stream), "stage event");
    return MOE_OK;
}

moe_status moe_forward(const moe_shape* shape, const void* x, const float* w_gate, const float* bias,
                       const void* w_in, const void* w_up, const void* w_out, void* out,
                       void* workspace, size_t ws_bytes, hipStream_t stream) {
    return moe_forward_timed(shape, x, w_gate, bias, w_in, w_up, w_out, out, workspace, ws_bytes, nullptr, stream);
}

moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const float* w_gate, const float* bias,
                               const void* w_in, const void* w_up, const void* w_out, void* out,
                               hipStream_t stream) {
    moe_status st = check_forward_args(shape, x, w_gate, bias, w_in, w_up, w_out, out);
    if (st != MOE_OK) return st;
    const size_t need = layout_of(*shape).total;
    if (need > kScratchBytes)
        return fail(MOE_ERR_WORKSPACE,
                    "this layer needs %zu bytes of scratch; the library's static scratch holds %zu "
                    "(use moe_forward with a caller workspace)", need, kScratchBytes);
    if (shape->T == 0) return MOE_OK;
    void* ws = nullptr;
    if ((st = scratch_of_current_device(&ws)) != MOE_OK) return st;
    return moe_forward_timed(shape, x, w_gate, bias, w_in, w_up, w_out, out, ws, kScratchBytes, nullptr, stream);
}

moe_status moe_workspace_layout(const moe_shape* shape, moe_workspace_parts* parts) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (!parts) return fail(MOE_ERR_NULL, "parts is NULL");
    const Layout L = layout_of(*shape);
    moe_workspace_parts p{};
    p.logit_parts = L.logits;
    p.logit_splits = gate_splits(shape->T, shape->H, shape->E, shape->dtype);
    p.topk_idx = L.topk_idx;
    p.topk_w = L.topk_w;
    p.counts = L.counts;
    p.offsets = L.offsets;
    p.sorted_token = L.sorted_token;
    p.row_of_pair = L.row_of_pair;
    p.h = L.h;
    p.y = L.y;
    p.total = L.total;
    *parts = p;
    return MOE_OK;
}

moe_status moe_capacity_rows(double capacity_factor, int64_t T, int32_t k, int32_t E, int32_t* rows) {
    if (!rows) return fail(MOE_ERR_NULL, "rows is NULL");
    if (!(capacity_factor > 0.0) || !(capacity_factor < 1e9))
        return fail(MOE_ERR_SHAPE, "capacity_factor = %g must be positive and finite", capacity_factor);
    if (T < 0 || k <= 0 || E <= 0) return fail(MOE_ERR_SHAPE, "T = %lld, k = %d, E = %d", (long long)T, k, E);
    // C = ceil(capacity_factor * (T * k) / E), in double; at least 1 (0 means no limit)
    const double c = std::ceil(capacity_factor * (double)(T * (long long)k) / (double)E);
    if (c >= 2147483647.0) return fail(MOE_ERR_SHAPE, "capacity %g does not fit int32", c);
    *rows = c < 1.0 ? 1 : (int32_t)c;
    return MOE_OK;
}

moe_status moe_router_stats(const moe_shape* shape, const float* logits, const float* bias,
                            const int32_t* counts, const int32_t* offsets, float* stats,
                            hipStream_t stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape& s = *shape;
    REQ(logits, "logits");
    OPT(bias, "bias");
    REQ(counts, "counts");
    REQ(stats, "stats");
    if (s.capacity > 0) REQ(offsets, "offsets");
    else OPT(offsets, "offsets");
    if (s.T == 0) return MOE_OK;
    (void)hipGetLastError();
    HIPCHK(launch_router_stats(logits, bias, counts, offsets, stats, s.T, s.E, s.k, s.capacity, stream),
           "router_stats");
    return MOE_OK;
}

const char* moe_status_str(moe_status status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
        case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: a size is out of range or inconsistent";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: outside this version's limits";
        case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: a pointer is not 16-byte aligned";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP call or launch failed";
        default: return "unknown moe_status";
    }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
