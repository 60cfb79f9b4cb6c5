/*
 * moe.h -- C ABI of the MI355X (gfx950) token-choice Mixture-of-Experts layer forward.
 *
 * Pages cited (by title and section):
 *   [FourStage]  "MoE显存与计算开销四阶段手算指南" (bjdmk.com.cn/news/5154310)
 *   [Principles] "MoE混合专家模型计算原理与推理部署实战解析" (sheratonhq.com/news/207562)
 *
 * The layer, per token t with hidden state x_t ([FourStage §2] four stages in order):
 *   logits  l_t = x_t @ W_g + b                         (gate projection, fp32)  [FourStage §2.1]
 *   top-k   the k experts with the largest l_t, slot 0 the largest, equal values
 *           to the lower index                                                   [FourStage §2.2]
 *   gates   softmax over all experts, then the k chosen renormalised to sum to 1:
 *           g_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0)                        [Principles §2.1-§2.2]
 *   group   per-expert counts, prefix sum, stable permutation to expert-major rows [Principles §5.1]
 *   experts SwiGLU: (SiLU(x W_gate) * (x W_up)) W_down                           [Principles §3.1]
 *           SiLU2 : SiLU(x W1) W2  (hidden -> d_ff -> hidden)                     [FourStage §2, §2.3]
 *           SiLU(z) = z / (1 + exp(-z)); no expert biases
 *   combine out_t = sum_j g_j * Expert_{e_j}(x_t), slot order j, fp32 accumulate,
 *           one rounding to the output type                                      [FourStage §2.4]
 *
 * Conventions shared by every entry point
 *   - Every array pointer is a DEVICE pointer (hipMalloc'd or equivalent), except the
 *     moe_shape pointer and moe_workspace_size's `bytes`, which are host pointers.
 *   - Arrays are dense, row-major, C-contiguous, with the shapes given below.  x, the
 *     expert weights, x_perm, y_perm and out use the element type `dtype`
 *     (fp32 or bf16); w_gate, bias, logits and topk_w are always fp32; index arrays
 *     are int32.  Expert weights are stacked [E, in, out] and used as h @ W.
 *   - Pair p = t*k + j is slot j of token t.  Grouped row r is a row of x_perm/y_perm.
 *   - Every device pointer must be 16-byte aligned.
 *   - Calls only enqueue work on `stream` (0 = the null stream) and return without
 *     synchronising.  Device faults surface at the caller's next synchronisation.
 *   - The caller owns every buffer.  Outputs are fully overwritten; inputs are only
 *     read; nothing is allocated, freed or kept between calls.  Calls on distinct
 *     workspaces and outputs are thread-safe.
 *   - Arguments are checked on the host before anything is enqueued.  A failed check
 *     returns its code, enqueues nothing, and sets the calling thread's
 *     moe_last_error() text.  T == 0 returns MOE_OK and enqueues nothing.
 *   - A failed kernel launch returns MOE_ERR_HIP with the HIP error text.
 *   - No C++ exception crosses this interface.
 *
 * Limits of this version: 1 <= E <= 256; 1 <= k <= min(E, 8); H % 8 == 0; F % 8 == 0;
 * T * k < 2^31; T*k*max(H,F) < 4e18 elements; x (T*H elements) and one expert matrix
 * with 128 extra rows ((H+128)*F and (F+128)*H elements) below 2 GiB each, since the
 * grouped GEMM reads them through buffer resources with 32-bit byte offsets and an
 * out-of-range marker at 2^31; for bf16 x and T > 256 the gate's weight planes
 * (3 * E * H rounded up to a multiple of 32, bf16) below 2 GiB too, for the same
 * reason (MOE_ERR_UNSUPPORTED otherwise).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,         /* a required pointer is NULL */
    MOE_ERR_SHAPE = 2,        /* a size is out of range or inconsistent */
    MOE_ERR_UNSUPPORTED = 3,  /* valid but outside this version's limits, or a bad enum/flag */
    MOE_ERR_ALIGN = 4,        /* a pointer is not 16-byte aligned */
    MOE_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than moe_workspace_size() */
    MOE_ERR_HIP = 6           /* a HIP call or kernel launch failed */
} moe_status;

/* element type of x, expert weights, x_perm, h, y_perm and out */
enum { MOE_F32 = 0, MOE_BF16 = 1 };
/* expert FFN form */
enum { MOE_FFN_SILU2 = 0, MOE_FFN_SWIGLU = 1 };

/* moe_shape.flags: routing variants.
 * MOE_FLAG_BIAS_SELECT_ONLY: the bias only picks the experts (l + b ranks them); the
 *   gates come from the unbiased logits l ([Principles §4.4], the auxiliary-loss-free
 *   balancing bias that takes no part in the output).
 * MOE_FLAG_NO_RENORM: the gates are the chosen experts' full-softmax probabilities,
 *   not renormalised over the k chosen ([FourStage §3] walk-through keeps them raw). */
#define MOE_FLAG_BIAS_SELECT_ONLY 0x1u
#define MOE_FLAG_NO_RENORM        0x2u

typedef struct {
    int64_t  T;          /* tokens (= batch * seq_len), >= 0 */
    int32_t  H;          /* hidden size */
    int32_t  E;          /* experts */
    int32_t  k;          /* experts per token (top_k) */
    int32_t  F;          /* expert intermediate size (d_ff) */
    int32_t  dtype;      /* MOE_F32 or MOE_BF16 */
    int32_t  ffn;        /* MOE_FFN_SILU2 or MOE_FFN_SWIGLU */
    uint32_t flags;      /* 0 or MOE_FLAG_* bits */
    int32_t  capacity;   /* rows per expert kept by moe_permute; 0 = no limit (dropless).
                            With C > 0 the pairs of expert e beyond its first C (in token
                            order) are dropped: they get no grouped row and add nothing
                            to the output ([Principles §4.3] capacity factor:
                            C = ceil(capacity_factor * T * k / E), see moe_capacity_rows). */
} moe_shape;

/* Per-expert row limit of a capacity factor, for moe_shape.capacity.  [Principles §4.3]
 * The page's capacity = capacity_factor * (total_tokens / num_experts), with the total
 * read as token-expert pairs T*k:  *rows = max(1, ceil(capacity_factor * (T*k) / E)),
 * evaluated in double precision.  capacity_factor must be positive and finite, T >= 0,
 * k, E > 0 (MOE_ERR_SHAPE otherwise; MOE_ERR_NULL if rows is NULL).  Host only. */
moe_status moe_capacity_rows(double capacity_factor, int64_t T, int32_t k, int32_t E, int32_t* rows);

/* Bytes of device workspace that moe_forward needs for `shape`; the same size is
 * enough for moe_permute and moe_grouped_ffn.  Host only; enqueues nothing. */
moe_status moe_workspace_size(const moe_shape* shape, size_t* bytes);

/* Where moe_forward keeps its intermediates inside the workspace: byte offsets from the
 * workspace base, for inspecting a finished call (tests, debugging).  After
 * moe_forward on `shape` has completed, the workspace holds
 *   logit_parts  [logit_splits][T][E] fp32: partial sums of x @ W_g over logit_splits
 *                consecutive ranges of H (no bias); top-k adds them in range order,
 *                then adds the bias once
 *   topk_idx     [T, k] int32, topk_w [T, k] fp32: the routing the layer used
 *   counts       [E] int32, offsets [E+1] int32, sorted_token [T*k] int32,
 *   row_of_pair  [T*k] int32: the grouping, as moe_permute defines them
 *   h            [offsets[E], F] dtype: first-projection output, grouped rows
 *   y            [offsets[E], H] dtype: second-projection output (y_perm)
 * total is moe_workspace_size().  The contents are undefined before the call ends or
 * after another call reuses the workspace.  Host only; enqueues nothing. */
typedef struct {
    size_t  logit_parts;
    int32_t logit_splits;
    int32_t reserved;
    size_t  topk_idx, topk_w, counts, offsets, sorted_token, row_of_pair, h, y, total;
} moe_workspace_parts;
moe_status moe_workspace_layout(const moe_shape* shape, moe_workspace_parts* parts);

/* Gate projection, top-k and gates.  [FourStage §2.1-§2.2], [Principles §2.1-§2.2, §2.4]
 *   x        [T, H] dtype, or NULL: then `logits` is an INPUT of fp32 logits (no bias)
 *   w_gate   [H, E] fp32 (ignored when x is NULL; may be NULL then)
 *   bias     [E] fp32 or NULL.  The ranking score is the single fp32 add l + b.
 *   logits   [T, E] fp32, required: the input when x is NULL; otherwise an output,
 *            x @ W_g in fp32 without the bias (top-k reads it back)
 *   topk_idx [T, k] int32 out: chosen experts, slot 0 the highest score; equal
 *            scores go to the lower index (-0 equals +0)
 *   topk_w   [T, k] fp32 out: gates of the chosen experts (see the flags)
 * The projection accumulates in fp32; bf16 x is widened exactly. */
moe_status moe_route(const moe_shape* shape, const void* x, const float* w_gate,
                     const float* bias, float* logits, int32_t* topk_idx, float* topk_w,
                     hipStream_t stream);

/* Group the T*k pairs by expert.  [FourStage §2.3], [Principles §5.1 steps 2-3]
 *   topk_idx     [T, k] int32 in, values in [0, E)
 *   x            [T, H] dtype, or NULL (then x_perm is not written)
 *   counts       [E] int32 out: pairs routed to each expert (before any capacity drop)
 *   offsets      [E+1] int32 out: first grouped row of each expert; offsets[E] = rows
 *                kept (T*k without a capacity)
 *   sorted_token [T*k] int32 out: token of grouped row r, for r < offsets[E] (rows of
 *                one expert in ascending token order); entries past offsets[E] unset
 *   row_of_pair  [T*k] int32 out: grouped row of pair p, or -1 if the pair was dropped
 *   x_perm       [T*k, H] dtype out or NULL: x_perm[r] = x[sorted_token[r]] (bit copy)
 *   workspace    device scratch of at least moe_workspace_size() bytes
 * Deterministic: the result does not depend on scheduling. */
moe_status moe_permute(const moe_shape* shape, const int32_t* topk_idx, const void* x,
                       int32_t* counts, int32_t* offsets, int32_t* sorted_token,
                       int32_t* row_of_pair, void* x_perm, void* workspace, size_t ws_bytes,
                       hipStream_t stream);

/* Every expert's FFN on its grouped rows, as grouped GEMMs in one pass per projection.
 * [FourStage §4.3] (one launch for all experts, driven by per-expert row offsets),
 * [Principles §3.1-§3.2]
 *   x_perm  [T*k, H] dtype: grouped rows; rows of expert e are [offsets[e], offsets[e+1])
 *   offsets [E+1] int32 (device), as written by moe_permute
 *   w_in    [E, H, F] dtype: W1 (SiLU2) or W_gate (SwiGLU)
 *   w_up    [E, H, F] dtype: W_up for SwiGLU; must be NULL for SiLU2
 *   w_out   [E, F, H] dtype: W2 / W_down
 *   y_perm  [T*k, H] dtype out: rows [0, offsets[E]) written
 * bf16: products accumulate in fp32; the intermediate h is rounded to bf16 once.
 * fp32: fp32 throughout. */
moe_status moe_grouped_ffn(const moe_shape* shape, const void* x_perm, const int32_t* offsets,
                           const void* w_in, const void* w_up, const void* w_out,
                           void* y_perm, void* workspace, size_t ws_bytes,
                           hipStream_t stream);

/* Gate-weighted combine back to token order.  [FourStage §2.4], [Principles §2.2]
 *   y_perm      [T*k, H] dtype
 *   row_of_pair [T*k] int32 (-1 = dropped pair, contributes nothing)
 *   topk_w      [T, k] fp32
 *   out         [T, H] dtype out: out[t] = sum_j topk_w[t,j] * y_perm[row_of_pair[t*k+j]],
 *               accumulated in fp32 in slot order, rounded once.  No atomics. */
moe_status moe_combine(const moe_shape* shape, const void* y_perm, const int32_t* row_of_pair,
                       const float* topk_w, void* out, hipStream_t stream);

/* The whole layer: route, group, grouped FFN, combine.  [FourStage §2], [Principles §6.1]
 * Same arguments and layouts as the stage calls; every intermediate lives in
 * `workspace` (moe_workspace_size() bytes).  The residual add is not part of it. */
moe_status moe_forward(const moe_shape* shape, const void* x, const float* w_gate,
                       const float* bias, const void* w_in, const void* w_up,
                       const void* w_out, void* out, void* workspace, size_t ws_bytes,
                       hipStream_t stream);

/* moe_forward without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, layouts and results as moe_forward; the intermediates
 * live in a static device scratch array of MOE_NOALLOC_SCRATCH_BYTES (256 MiB) inside
 * the library, one per GPU, held until the process ends.  Nothing is allocated or
 * freed by the call.  A layer whose moe_workspace_size() exceeds the scratch returns
 * MOE_ERR_WORKSPACE (enqueuing nothing).  Every call on one GPU uses that GPU's one
 * scratch array, so calls that overlap on a GPU (concurrent streams or threads) race
 * and give undefined results: serialise them.  The call itself clears what its kernels
 * need zeroed; nothing depends on an earlier call's contents. */
#define MOE_NOALLOC_SCRATCH_BYTES (256u << 20)
moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const float* w_gate,
                               const float* bias, const void* w_in, const void* w_up,
                               const void* w_out, void* out, hipStream_t stream);

/* Router statistics of one batch ([Principles §4.2, §5.2]), from fp32 logits (no bias)
 * and the per-expert counts:
 *   stats [E + 4] fp32 out: stats[e] = P_e, the mean over tokens of expert e's softmax
 *   probability (of l + b), stats[E] = balance = E * sum_e f_e P_e with f_e = counts[e] /
 *   (T*k), stats[E+1] = entropy (nats) of f, stats[E+2] = mean top-1 probability,
 *   stats[E+3] = fraction of pairs dropped by the capacity (0 without one).
 *   offsets may be NULL when shape->capacity == 0. */
moe_status moe_router_stats(const moe_shape* shape, const float* logits, const float* bias,
                            const int32_t* counts, const int32_t* offsets, float* stats,
                            hipStream_t stream);

/* moe_forward with timing events, for benchmarks.  `events` is NULL (then this is
 * moe_forward) or MOE_STAGE_EVENTS events of the caller, created with timing enabled,
 * which are recorded on `stream` at the stage boundaries:
 *   [0] before the gate projection
 *   [1] after top-k and gates (the routing stage, [FourStage §2.1-§2.2])
 *   [2] after the grouping (histogram, offsets, maps, the GEMM tile list, [Principles §5.1]),
 *       i.e. just before the launch of the first expert projection (w_in, and w_up)
 *   [3] between the two expert projections (before the w_out launch)
 *   [4] after the second projection
 *   [5] after the combine ([FourStage §2.4])
 * so hipEventElapsedTime between neighbours gives each stage's duration, and [2]-[3],
 * [3]-[4] each projection kernel's.  A NULL entry is MOE_ERR_NULL.  Nothing is kept
 * after the call returns. */
#define MOE_STAGE_EVENTS 6
moe_status moe_forward_timed(const moe_shape* shape, const void* x, const float* w_gate,
                             const float* bias, const void* w_in, const void* w_up,
                             const void* w_out, void* out, void* workspace, size_t ws_bytes,
                             const hipEvent_t* events, hipStream_t stream);

/* Static text for a status code. */
const char* moe_status_str(moe_status status);

/* Detail of the calling thread's most recent non-OK return ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
