/*
 * moe.h - C ABI of the MI355X (gfx950) sparse Mixture-of-Experts layer forward.
 *
 * The library computes the forward pass of one sparse MoE layer:
 *   router linear -> softmax / top-k -> optional per-expert capacity with token
 *   dropping -> dispatch into an expert-sorted permutation -> per-expert FFN
 *   (grouped GEMM) -> routing-weighted combine (+ optional shared expert).
 *
 * Sources, cited by page and section:
 *   [mlqm]   www.mlqm.cn/news/130088: §3.1 Router (logits = h W_r, softmax, top-k),
 *            §3.3 Gate (w_i = p_i / (p_i + p_j), -inf masking), §4.2 model code.
 *   [rkmt]   "大模型MoE架构揭秘：为什么总参数≠激活参数": §2.3 expert capacity (T*k)/E,
 *            overflow tokens dropped.
 *   [200B-5] "[从零训练一个200B大语言模型] 5/25：MoE怎样用一部分参数，完成一次计算？":
 *            "谁来决定请哪几个专家？" (router, top-k, weighted mixture of the selected
 *            experts' outputs), "共享专家，给每个token都走的一条路" (shared expert).
 *   [cnnet]  "MoE混合专家架构原理与工程实践：解密大模型稀疏计算真相": stacked ("fused")
 *            expert weights sliced by index, batching the tokens of one expert.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless stated otherwise.  The caller allocates and
 *     owns every input, output and workspace buffer; the library never allocates,
 *     frees, copies to or from the host, or synchronises.
 *   - Every call validates its arguments on the host first.  On any error it returns
 *     a non-zero status before launching anything, so no output is touched.
 *     moe_last_error() then describes the problem (thread-local string).
 *   - On MOE_OK all work has been enqueued on `stream` (in stream order); results are
 *     visible after the caller synchronises the stream.  A kernel launch failure
 *     returns MOE_EHIP (work enqueued before it may have run).
 *   - Matrices are row-major and contiguous.  Expert weights use the nn.Linear
 *     layout [out, in]: w_gate / w_up are [G, F, d] and w_down is [G, d, F]; bf16
 *     weights may instead be stored in the packed layout made by moe_pack_weights
 *     (same shape and size, see moe_layout_t).
 *   - dtype MOE_BF16: x, w_r and expert weights are bfloat16; products are exact in
 *     fp32 and accumulate in fp32; the hidden activation of the expert is rounded to
 *     bf16 once.  MOE_F32: everything is fp32.  Logits, routing weights and the
 *     per-row expert outputs y are always fp32.
 *   - Requirements: T >= 0 (T == 0 is a no-op), d >= 1, 1 <= E <= 1024,
 *     1 <= k <= E, F >= 1; for MOE_BF16 expert FFNs, d and F must be multiples of 64,
 *     the hidden states x (T x d bf16) and one expert matrix (F x d bf16) must each stay
 *     below 2 GiB (at d = 4096: up to 262143 tokens per call; the hidden activation and
 *     the expert outputs, which grow with T k F, have no such limit), and MOE_BF16
 *     routing with d not a multiple of 32 takes at most 888 experts (MOE_EUNSUPPORTED
 *     otherwise).  Pointers must be 16-byte aligned.
 *   - Calls on the same stream are ordered; concurrent calls on different streams
 *     share no library state.
 *   - Graph capture: the compute calls enqueue kernels only (no allocation, memset,
 *     copy or synchronisation), so they can be captured into a HIP graph on the
 *     caller's stream.  Make one uncaptured call with the same sizes first: the first
 *     call of a size may set a kernel's dynamic-LDS attribute (a host-side call).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every enum below also lists a smallest and a largest int32 value (the *_RANGE_MIN_ and
 * *_RANGE_MAX_ entries, never valid arguments): every int a C caller passes is then a value
 * of the type, and the library can reject an out-of-range one with MOE_EINVAL (in C++ an
 * enum object may not hold a value outside the range of its enumerators). */
typedef enum {
  MOE_STATUS_RANGE_MIN_ = -2147483647 - 1,
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* null required pointer, bad size or enum */
  MOE_EUNSUPPORTED = 2,  /* valid but unsupported shape (e.g. bf16 d % 64 != 0) */
  MOE_EWORKSPACE = 3,    /* workspace smaller than the *_workspace_bytes() figure */
  MOE_EHIP = 4,          /* a HIP launch or runtime call failed */
  MOE_STATUS_RANGE_MAX_ = 2147483647
} moe_status_t;

typedef enum { MOE_DTYPE_RANGE_MIN_ = -2147483647 - 1, MOE_F32 = 0, MOE_BF16 = 1, MOE_DTYPE_RANGE_MAX_ = 2147483647 } moe_dtype_t;
typedef enum { MOE_ACT_RANGE_MIN_ = -2147483647 - 1, MOE_ACT_GELU = 0, MOE_ACT_SWIGLU = 1, MOE_ACT_RANGE_MAX_ = 2147483647 } moe_act_t;
/* Routing weights of the selected experts:
 *   MOE_WEIGHTS_RENORMALIZED  w_j = p_{s_j} / sum_{i<k} p_{s_i}   ([mlqm] §3.3, §4.2)
 *   MOE_WEIGHTS_SOFTMAX       w_j = p_{s_j}, the softmax probabilities themselves
 *                             ("MoE混合专家架构原理与工程实践…" §3.2: output = p1 e1 + p2 e2) */
typedef enum {
  MOE_WEIGHTS_RANGE_MIN_ = -2147483647 - 1,
  MOE_WEIGHTS_RENORMALIZED = 0,
  MOE_WEIGHTS_SOFTMAX = 1,
  MOE_WEIGHTS_RANGE_MAX_ = 2147483647
} moe_weights_t;
/* Order in which slots claim expert capacity ([rkmt] §2.3 keeps what fits, drops the rest):
 *   MOE_PRIORITY_TOKEN  ascending token, then slot: the earliest tokens are kept
 *   MOE_PRIORITY_SLOT   all first choices, then all second choices, ...; ascending token
 *                       within one slot position (first choices are never displaced) */
typedef enum {
  MOE_PRIORITY_RANGE_MIN_ = -2147483647 - 1,
  MOE_PRIORITY_TOKEN = 0,
  MOE_PRIORITY_SLOT = 1,
  MOE_PRIORITY_RANGE_MAX_ = 2147483647
} moe_priority_t;
/* What happens to a slot beyond its expert's capacity ([rkmt] §2.3: dropped, or sent to
 * the next-best expert):
 *   MOE_OVERFLOW_DROP     the slot contributes zero
 *   MOE_OVERFLOW_REROUTE  after the router's choices have claimed capacity, the overflowed
 *                         slots, in priority order, each move to the token's best expert
 *                         (by logit, lowest index on ties) outside its top-k and its
 *                         earlier re-routes that still has room, else are dropped; a moved
 *                         slot keeps its routing weight */
typedef enum {
  MOE_OVERFLOW_RANGE_MIN_ = -2147483647 - 1,
  MOE_OVERFLOW_DROP = 0,
  MOE_OVERFLOW_REROUTE = 1,
  MOE_OVERFLOW_RANGE_MAX_ = 2147483647
} moe_overflow_t;
/* Storage order of the bf16 expert weights (w_gate, w_up, w_down and the shared expert's):
 *   MOE_LAYOUT_LINEAR  the nn.Linear layout [G, N, K], K contiguous
 *   MOE_LAYOUT_PACKED  the same values reordered by moe_pack_weights into MFMA operand
 *                      fragments (same size); the expert FFN then reads each 16 x 32
 *                      fragment as one contiguous KiB.  The results are bit-identical to
 *                      the linear layout's. */
typedef enum {
  MOE_LAYOUT_RANGE_MIN_ = -2147483647 - 1,
  MOE_LAYOUT_LINEAR = 0,
  MOE_LAYOUT_PACKED = 1,
  MOE_LAYOUT_RANGE_MAX_ = 2147483647
} moe_layout_t;

/* Explicit tile shape of the bf16 grouped expert GEMM (host struct; for tuning and tests).
 *   rows   rows per M-tile: 32, 64, 128, 192 or 256; 0 = chosen from the sizes (the
 *          expected rows per routed expert: capacity if set, else 1.6x the mean load)
 *   waves  waves per workgroup: 4, 8 or 16; 0 = 8
 * 192-row tiles exist with 8 waves only; with another explicit wave count and rows = 0
 * the automatic height is raised from 192 to 256.  Any other value, or 192 rows with an
 * explicit 4 or 16 waves, is MOE_EUNSUPPORTED.  The tile shape changes the schedule of the
 * work, never a result bit.  fp32 layers have one tile shape and ignore it. */
typedef struct moe_tile {
  int32_t rows;
  int32_t waves;
} moe_tile_t;

/* Static description of a status code (host). */
const char* moe_status_string(moe_status_t s);
/* Message of the last failing call on this host thread ("" if none). */
const char* moe_last_error(void);

/*
 * moe_route - router logits, top-k selection and routing weights.
 *   [mlqm] §3.1: logits z = h W_r (+ per-expert offset b), softmax over E experts,
 *   keep the k best.  [mlqm] §3.3 / §4.2: the kept probabilities are renormalised,
 *   w_j = p_{s_j} / sum_i p_{s_i} = exp(z_{s_j} - z_{s_0}) / sum_i exp(z_{s_i} - z_{s_0}).
 *   x        [T, d]   dtype dt
 *   w_r      [d, E]   dtype dt
 *   bias     [E] fp32 or NULL (no offsets)
 *   topk_idx [T, k] int32 out: expert of slot j, slots ordered by descending logit;
 *            equal logits are ordered by ascending expert index
 *   weights  moe_weights_t: how the selected probabilities become routing weights
 *   topk_w   [T, k] fp32 out: routing weights (sum to 1 per token when renormalised)
 *   logits   [T, E] fp32 out: the router logits (fp32 accumulation)
 *   ws       device workspace of moe_route_workspace_bytes(T, d, E, dt) bytes (may be NULL
 *            when that is 0): with few tokens the contraction over d is split across
 *            workgroups and the partial logits are added in a fixed order
 * Deterministic: identical inputs and sizes give identical bits.
 */
size_t moe_route_workspace_bytes(int64_t T, int64_t d, int32_t E, moe_dtype_t dt);
moe_status_t moe_route(const void* x, const void* w_r, const float* bias, moe_dtype_t dt,
                       int64_t T, int64_t d, int32_t E, int32_t k, moe_weights_t weights,
                       int32_t* topk_idx, float* topk_w, float* logits, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/*
 * moe_capacity - per-expert capacity from a capacity factor (host, pure).
 *   [rkmt] §2.3: each of E experts takes (T*k)/E slots, e.g. (1024*2)/16 = 128; the
 *   DeepSpeed-MoE block of "MoE混合专家架构原理与工程实践…" §4.2 scales that by a capacity
 *   factor (1.2 in training, 2.0 at inference) with a floor (min_capacity 4).
 *   Returns max(min_capacity, ceil(factor * T * k / E)), the product evaluated left to
 *   right in double precision, clamped to 2^31 - 1.  The result is meant for the
 *   `capacity` argument of moe_dispatch / moe_layer_args_t, where <= 0 means unlimited.
 *   Invalid arguments (T < 0, k < 1, E < 1, non-finite factor) return 0 (unlimited).
 */
int64_t moe_capacity(int64_t T, int32_t k, int32_t E, double factor, int64_t min_capacity);

/* Workspace bytes moe_dispatch needs for T tokens, E experts, k slots, any policy
 * (host, pure). */
size_t moe_dispatch_workspace_bytes(int64_t T, int32_t E, int32_t k);

/*
 * moe_dispatch - per-expert counts, capacity, expert-sorted permutation.
 *   [rkmt] §2.3: expert e accepts at most `capacity` slots; the overflow is dropped
 *   (zero contribution) or re-routed, see moe_priority_t and moe_overflow_t.
 *   topk_idx  [T, k] int32 in  (values in [0, E); other values are undefined behaviour).
 *             A row may name one expert in several slots: each such slot is its own
 *             row of that expert (in priority order), as any other slot.
 *   logits    [T, E] fp32 in  (the router logits; read only for MOE_OVERFLOW_REROUTE with
 *             capacity > 0, may be NULL otherwise)
 *   capacity  <= 0: unlimited
 *   priority  moe_priority_t; overflow  moe_overflow_t
 *   counts    [E] int32 out: slots that selected e (demand, before capacity)
 *   offsets   [E+1] int32 out: exclusive prefix sum of the rows each expert computes
 *             (min(counts, capacity), plus re-routed arrivals)
 *   perm      [T*k] int32 out: perm[r] = t*k + j for each row r < offsets[E]; the rows
 *             of one expert are its router-chosen slots in priority order, then the
 *             slots re-routed to it in re-route order; entries >= offsets[E] untouched
 *   inv       [T*k] int32 out: row of slot (t, j), or -1 when the slot was dropped
 *   n_dropped [1] int32 out: number of dropped slots
 *   ws        device workspace of at least moe_dispatch_workspace_bytes(T, E, k) bytes
 * Integer-only and deterministic (bit-identical across runs).  Re-routing walks the
 * overflow sequentially in one wave (it is a greedy choice in priority order).
 */
moe_status_t moe_dispatch(const int32_t* topk_idx, const float* logits, int64_t T, int32_t E, int32_t k,
                          int64_t capacity, moe_priority_t priority, moe_overflow_t overflow,
                          int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                          int32_t* n_dropped, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_pack_weights - reorder stacked bf16 expert weights for the expert FFN.
 *   [cnnet]: the experts' weights are stacked in one tensor and sliced by expert index;
 *   this is a one-time change of that tensor's storage order, done when the weights are
 *   loaded, not part of a forward pass.
 *   w       [G, N, K] bf16 in, nn.Linear layout (w_gate / w_up: N = F, K = d;
 *           w_down: N = d, K = F; a shared expert's weights with G = 1)
 *   packed  [G, N, K] bf16 out (same size, must not overlap w): 16-byte chunk
 *           c = ((g * N/16 + i) * K/32 + j) * 64 + l holds w[g][16 i + l % 16][32 j + 8 (l / 16) + 0..7]
 *   Requirements: G >= 1, N % 16 == 0 and K % 32 == 0 (MOE_EUNSUPPORTED otherwise).
 * Pure data movement, deterministic.
 */
moe_status_t moe_pack_weights(const void* w, void* packed, int64_t G, int64_t N, int64_t K,
                              hipStream_t stream);

/* Workspace bytes moe_expert_ffn needs (host, pure; tile as for moe_expert_ffn, may be
 * NULL; 0 for an invalid size or tile). */
size_t moe_expert_ffn_workspace_bytes(int64_t max_rows, int32_t G, int64_t d, int64_t F,
                                      moe_act_t act, moe_dtype_t dt, const moe_tile_t* tile);

/*
 * moe_expert_ffn - every group's FFN over its rows (grouped GEMM).
 *   [cnnet]: experts stacked in one tensor and sliced by index; the rows routed to one
 *   expert are computed together.  GeLU expert: y = W2 gelu(W1 x) with w_gate = W1
 *   [G,F,d], w_down = W2 [G,d,F], w_up = NULL.  SwiGLU expert:
 *   y = Wd (silu(Wg x) * (Wu x)) with w_gate = Wg, w_up = Wu [G,F,d], w_down = Wd.
 *   x        [n_x, d] dtype dt (bf16: below 2 GiB; without perm n_x >= max_rows is checked,
 *            with perm every row perm[r] / k it names must lie inside those 2 GiB)
 *   perm     NULL: row r reads x[r];  else row r reads x[perm[r] / k]
 *   offsets  [G+1] int32 (device): group g owns rows [offsets[g], offsets[g+1]),
 *            non-decreasing, offsets[0] >= 0.  Rows at or beyond max_rows are ignored.
 *   max_rows host upper bound of offsets[G] (sizes the launch and the workspace)
 *   layout   moe_layout_t of w_gate, w_up and w_down (MOE_LAYOUT_PACKED: bf16 only)
 *   y        [max_rows, d] fp32 out: y[r] for r < min(offsets[G], max_rows)
 *   tile     host pointer to an explicit tile shape (moe_tile_t), or NULL for the
 *            automatic choice
 *   ws       device workspace of moe_expert_ffn_workspace_bytes(..., tile) bytes
 */
moe_status_t moe_expert_ffn(const void* x, const int32_t* perm, int32_t k,
                            const int32_t* offsets, int32_t G, int64_t max_rows,
                            int64_t d, int64_t F, moe_act_t act, moe_dtype_t dt,
                            moe_layout_t layout, const void* w_gate, const void* w_up, const void* w_down,
                            float* y, const moe_tile_t* tile, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * moe_combine - routing-weighted sum of the selected experts' outputs.
 *   [200B-5] "谁来决定请哪几个专家？": out = sum_j w_j * Expert_j(x) (the worked example
 *   0.75*[0.8,0.2,-0.4] + 0.25*[0.4,0.6,0.8] = [0.7,0.3,-0.1]); "共享专家…": the
 *   shared expert's result is added.  A dropped slot (inv < 0) adds nothing and the
 *   other weights are not renormalised.  Accumulates in fp32, rounds once to out_dt.
 *   y       [y_rows, d] fp32 expert outputs in row order
 *   inv     [T, k] int32 row of each slot, -1 = dropped (rows >= y_rows are ignored)
 *   topk_w  [T, k] fp32 routing weights
 *   shared  [T, d] fp32 shared-expert output, or NULL
 *   out     [T, d] out, dtype out_dt
 */
moe_status_t moe_combine(const float* y, int64_t y_rows, const int32_t* inv,
                         const float* topk_w, const float* shared, int64_t T, int64_t d,
                         int32_t k, moe_dtype_t out_dt, void* out, hipStream_t stream);

/* Number of floats moe_routing_stats writes for E experts. */
#define MOE_STATS_FLOATS(E) (5 + (E))

/* Workspace bytes moe_routing_stats needs for T tokens (host, pure). */
size_t moe_routing_stats_workspace_bytes(int64_t T);

/*
 * moe_routing_stats - load-balance terms and monitoring metrics of one batch.
 *   With u_e = counts[e] / T (the fraction of tokens that selected e; sum_e u_e = k):
 *   stats[0] balance ratio std(u) / (mean(u) + 1e-8), std with Bessel's correction
 *            ([mlqm] §4.2 code); stats[1] = lambda_balance * stats[0] ([mlqm] §3.1, 0.01)
 *   stats[2] L_aux = lambda_aux * (std(u) + gamma_aux * max(u))
 *            ("MoE混合专家架构原理与工程实践…" §3.2: lambda 0.01, gamma 100)
 *   stats[3] router entropy: mean over tokens of -sum_e p_e ln p_e, p = softmax(logits)
 *   stats[4] token drop rate n_dropped / (T k)                ("大模型MoE架构揭秘…" §6.1)
 *   stats[5 + e] utilization ratio counts[e] / (T k)            ("大模型MoE架构揭秘…" §6.1)
 *   logits [T, E] fp32, counts [E] int32 (demand, as written by moe_dispatch),
 *   n_dropped [1] int32 or NULL (0), stats [MOE_STATS_FLOATS(E)] fp32 out.
 *   Reductions run in a fixed order in double precision: bit-reproducible.
 */
moe_status_t moe_routing_stats(const float* logits, const int32_t* counts, const int32_t* n_dropped,
                               int64_t T, int32_t E, int32_t k, float lambda_balance, float lambda_aux,
                               float gamma_aux, float* stats, void* ws, size_t ws_bytes, hipStream_t stream);

/* Arguments of the whole layer (host struct; pointers inside are device pointers). */
typedef struct moe_layer_args {
  int32_t dt;            /* moe_dtype_t: activations and weights */
  int32_t act;           /* moe_act_t */
  int32_t out_dt;        /* moe_dtype_t of `out`: MOE_F32 (0, the fp32 accumulator rounded
                            once) or MOE_BF16 (rounded once to bf16) */
  int32_t weights;       /* moe_weights_t (0: renormalised) */
  int32_t priority;      /* moe_priority_t (0: token order) */
  int32_t overflow;      /* moe_overflow_t (0: drop) */
  int32_t layout;        /* moe_layout_t of the expert weights, routed and shared (0: linear;
                            packed needs dt = MOE_BF16) */
  int64_t T, d, F;
  int32_t E, k;
  int64_t capacity;      /* <= 0: unlimited */
  const void* x;         /* [T, d] */
  const void* w_r;       /* [d, E] */
  const float* bias;     /* [E] router offsets or NULL */
  const void* w_gate;    /* [E, F, d] */
  const void* w_up;      /* [E, F, d], NULL for GeLU */
  const void* w_down;    /* [E, d, F] */
  const void* s_gate;    /* shared expert [F, d], or NULL for none */
  const void* s_up;      /* [F, d] (SwiGLU) or NULL */
  const void* s_down;    /* [d, F] */
  void* out;             /* [T, d] out, dtype out_dt */
  /* Optional outputs; NULL keeps them inside the workspace. */
  int32_t* topk_idx;     /* [T, k] */
  float* topk_w;         /* [T, k] */
  float* logits;         /* [T, E] */
  int32_t* counts;       /* [E] */
  int32_t* offsets;      /* [E+1] */
  int32_t* perm;         /* [T*k] */
  int32_t* inv;          /* [T*k] */
  int32_t* n_dropped;    /* [1] */
  void* ws;              /* device workspace */
  size_t ws_bytes;
  /* Optional measurement hook: NULL, or MOE_STAGE_EVENTS hipEvent_t handles created by
     the caller.  Event i is recorded on `stream` right after stage boundary i:
     0 start, 1 route, 2 dispatch, 3 FFN schedule, 4 FFN up-projection (gate/up GEMM),
     5 FFN down-projection, 6 combine.  The library only records them. */
  void* const* stage_events;
  /* Optional routing statistics (moe_routing_stats layout), computed after dispatch:
     NULL, or MOE_STATS_FLOATS(E) floats, with the three coefficients below. */
  float* stats;
  float lambda_balance, lambda_aux, gamma_aux;
  /* Explicit tile shape of the expert FFN (moe_tile_t); all zero = automatic. */
  moe_tile_t tile;
} moe_layer_args_t;

#define MOE_STAGE_EVENTS 7

/* Workspace bytes moe_layer_forward needs for these arguments (host, pure). */
size_t moe_layer_workspace_bytes(const moe_layer_args_t* a);

/* How moe_layer_forward will run the expert FFN for these arguments (host, pure). */
typedef struct moe_ffn_plan {
  int32_t tile_rows;     /* rows per M-tile of the grouped GEMMs (fp32 layers: 64) */
  int32_t tile_waves;    /* waves per workgroup (fp32 layers: 4) */
  int32_t down_splits;   /* the down projection's contraction is split this many ways */
} moe_ffn_plan_t;
/* Fills *plan; MOE_EINVAL / MOE_EUNSUPPORTED for arguments the forward would reject on
 * their sizes, enums or tile (pointers are not examined). */
moe_status_t moe_layer_plan(const moe_layer_args_t* a, moe_ffn_plan_t* plan);

/*
 * moe_layer_forward - the whole layer on one stream:
 *   route -> dispatch -> grouped expert FFN (the shared expert runs as one more group
 *   over all T tokens) -> combine.  No host synchronisation inside.
 *   Result: out[t] = shared(x_t) + sum_{kept j} w_{t,j} * Expert_{idx_{t,j}}(x_t).
 */
moe_status_t moe_layer_forward(const moe_layer_args_t* a, hipStream_t stream);

/* Size of the fixed device scratch of moe_layer_forward_noalloc, per GPU. */
#define MOE_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * moe_layer_forward_noalloc - moe_layer_forward for callers that cannot allocate device
 *   memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 *   hipMalloc): the same kernels and results (bit-identical), but the workspace is a
 *   fixed array of MOE_SCRATCH_BYTES inside the library, one per GPU, held until the
 *   process ends.  a->ws and a->ws_bytes are ignored; the caller still passes every input
 *   and output.  The call allocates and frees nothing.
 *   Limit: moe_layer_workspace_bytes(a) <= MOE_SCRATCH_BYTES, else MOE_EWORKSPACE before
 *   any launch (at d = 4096, F = 14336, k = 2 about 700 tokens per call: decode-sized
 *   batches).  Invalid arguments: as moe_layer_forward.  The first call on a device looks
 *   up that device's array (hipGetSymbolAddress; MOE_EHIP if that fails).
 *   Every call on one GPU uses the same array, and each call overwrites it: calls that
 *   overlap in time on one GPU (other streams, or other host threads without ordering)
 *   race and give undefined results.  Calls ordered on one stream are safe.
 */
moe_status_t moe_layer_forward_noalloc(const moe_layer_args_t* a, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
