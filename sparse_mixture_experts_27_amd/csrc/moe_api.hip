// C-ABI entry points: host-side validation, workspace carving, launches.
// The layer forward chains route -> dispatch -> grouped FFN -> combine on one stream
// ([mlqm] §4.2 forward steps 1-4; [200B-5] "谁来决定请哪几个专家？" and "共享专家…").
#include "moe_common.h"

#include <cmath>
#include <mutex>
#include <map>
#include <utility>

namespace moe {

namespace {
thread_local char g_last_error[512] = "";
}

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

moe_status_t fail(moe_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

moe_status_t check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

void set_max_dynamic_smem(const void* func, size_t bytes) {
  // the attribute is a per-device cap: raise it whenever a launch needs more than any
  // earlier one on this device (a later, larger problem must not inherit a smaller cap)
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, size_t> cap;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return;
  std::lock_guard<std::mutex> lk(mu);
  size_t& c = cap[{dev, func}];
  if (bytes > c) {
    if (hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes)) == hipSuccess)
      c = bytes;
  }
}

namespace {

bool valid_dt(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }
bool valid_act(int a) { return a == MOE_ACT_GELU || a == MOE_ACT_SWIGLU; }

moe_status_t check_layout(int layout, int dt) {
  if (layout != MOE_LAYOUT_LINEAR && layout != MOE_LAYOUT_PACKED)
    return fail(MOE_EINVAL, "weight layout %d is not MOE_LAYOUT_LINEAR or MOE_LAYOUT_PACKED", layout);
  if (layout == MOE_LAYOUT_PACKED && dt != MOE_BF16)
    return fail(MOE_EINVAL, "the packed weight layout is defined for bf16 weights only");
  return MOE_OK;
}

moe_status_t check_route_args(const void* x, const void* w_r, int dt, int64_t T, int64_t d, int E, int k,
                              const void* topk_idx, const void* topk_w, const void* logits) {
  if (!valid_dt(dt)) return fail(MOE_EINVAL, "dtype %d is not MOE_F32 or MOE_BF16", dt);
  if (T < 0 || T > (int64_t{1} << 31) - 1) return fail(MOE_EINVAL, "T=%lld out of range", (long long)T);
  if (d < 1) return fail(MOE_EINVAL, "d=%lld must be >= 1", (long long)d);
  if (E < 1 || E > kMaxExperts) return fail(MOE_EINVAL, "E=%d must be in [1, %d]", E, kMaxExperts);
  if (k < 1 || k > E) return fail(MOE_EINVAL, "k=%d must be in [1, E=%d]", k, E);
  if (T * k > (int64_t{1} << 31) - 1) return fail(MOE_EINVAL, "T*k exceeds 2^31-1");
  if (route_lds_bytes(d, E, dt) > kMaxLdsBytes)
    return fail(MOE_EUNSUPPORTED, "routing %d experts with d=%lld needs %zu bytes of LDS per workgroup (most %zu); "
                "bf16 routing with d not a multiple of 32 supports at most 888 experts",
                E, (long long)d, route_lds_bytes(d, E, dt), kMaxLdsBytes);
  if (T > 0 && (!x || !w_r || !topk_idx || !topk_w || !logits))
    return fail(MOE_EINVAL, "moe_route: null required pointer");
  if (T > 0 && (!aligned16(x) || !aligned16(w_r))) return fail(MOE_EINVAL, "x and w_r must be 16-byte aligned");
  return MOE_OK;
}

// The bf16 kernels address the hidden states x (rows gathered anywhere in it) and one
// expert's weights with 32-bit byte offsets from their start, so each must stay below 2 GiB;
// the hidden activation H is addressed from each tile's first row and has no such limit.
moe_status_t check_bf16_operands(int64_t x_rows, int64_t d, int64_t F) {
  constexpr int64_t kMaxOperand = (int64_t{1} << 31) - 1;
  if (x_rows * d * 2 > kMaxOperand)
    return fail(MOE_EUNSUPPORTED, "bf16 hidden states x must stay below 2 GiB (%lld rows x d=%lld); "
                "split the batch", (long long)x_rows, (long long)d);
  if (F * d * 2 > kMaxOperand)
    return fail(MOE_EUNSUPPORTED, "one bf16 expert matrix must stay below 2 GiB (F=%lld d=%lld)", (long long)F,
                (long long)d);
  return MOE_OK;
}

// An explicit tile shape must name a kernel (moe_tile_t); NULL or zeros = automatic.
moe_status_t check_tile(const moe_tile_t* t) {
  if (!t) return MOE_OK;
  const bool rows_ok = t->rows == 0 || t->rows == 32 || t->rows == 64 || t->rows == 128 || t->rows == 192 ||
                       t->rows == 256;
  const bool waves_ok = t->waves == 0 || t->waves == 4 || t->waves == 8 || t->waves == 16;
  if (!rows_ok || !waves_ok || (t->rows == 192 && t->waves != 0 && t->waves != 8))
    return fail(MOE_EUNSUPPORTED, "no expert FFN kernel for a tile of %d rows and %d waves "
                "(rows 32/64/128/192/256, waves 4/8/16, 192 rows with 8 waves only; 0 = automatic)",
                t->rows, t->waves);
  return MOE_OK;
}
int tile_rows_of(const moe_tile_t* t) { return t ? t->rows : 0; }
int tile_waves_of(const moe_tile_t* t) { return t ? t->waves : 0; }

moe_status_t check_ffn_args(const void* x, const int32_t* perm, const int32_t* offsets, int G, int64_t max_rows, int64_t d,
                            int64_t F, int act, int dt, const void* w_gate, const void* w_up,
                            const void* w_down, const void* y) {
  if (!valid_dt(dt)) return fail(MOE_EINVAL, "dtype %d is not MOE_F32 or MOE_BF16", dt);
  if (!valid_act(act)) return fail(MOE_EINVAL, "activation %d is not GeLU or SwiGLU", act);
  if (G < 1 || G > (1 << 20)) return fail(MOE_EINVAL, "G=%d out of range", G);
  if (max_rows < 0 || max_rows > (int64_t{1} << 31) - 1) return fail(MOE_EINVAL, "max_rows out of range");
  if (d < 1 || F < 1) return fail(MOE_EINVAL, "d and F must be >= 1");
  if (dt == MOE_BF16 && (d % 64 != 0 || F % 64 != 0))
    return fail(MOE_EUNSUPPORTED, "bf16 expert FFN needs d and F multiples of 64 (d=%lld F=%lld)",
                (long long)d, (long long)F);
  if (dt == MOE_BF16) {
    // without a permutation row r reads x[r]: x holds max_rows rows; with one, the rows of
    // x it names must lie inside the first 2 GiB of x (its row count is not an argument)
    if (moe_status_t st = check_bf16_operands(perm ? 0 : max_rows, d, F)) return st;
  }
  if (!x || !offsets || !w_gate || !w_down || !y) return fail(MOE_EINVAL, "moe_expert_ffn: null required pointer");
  if (act == MOE_ACT_SWIGLU && !w_up) return fail(MOE_EINVAL, "SwiGLU needs w_up");
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_down) || (w_up && !aligned16(w_up)) || !aligned16(y))
    return fail(MOE_EINVAL, "x, weights and y must be 16-byte aligned");
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: unsupported shape";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
    case MOE_EHIP: return "MOE_EHIP: HIP runtime error";
    default: break;
  }
  return "unknown moe_status_t";
}

const char* moe_last_error(void) { return g_last_error; }

size_t moe_route_workspace_bytes(int64_t T, int64_t d, int32_t E, moe_dtype_t dt) {
  if (T < 0 || d < 1 || E < 1 || !valid_dt(dt)) return 0;
  return route_ws_bytes(T, d, E, dt);
}

moe_status_t moe_route(const void* x, const void* w_r, const float* bias, moe_dtype_t dt, int64_t T, int64_t d,
                       int32_t E, int32_t k, moe_weights_t weights, int32_t* topk_idx, float* topk_w, float* logits,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  if (moe_status_t st = check_route_args(x, w_r, dt, T, d, E, k, topk_idx, topk_w, logits)) return st;
  if (weights != MOE_WEIGHTS_RENORMALIZED && weights != MOE_WEIGHTS_SOFTMAX)
    return fail(MOE_EINVAL, "weights mode %d invalid", weights);
  const size_t need = route_ws_bytes(T, d, E, dt);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(MOE_EWORKSPACE, "route needs %zu workspace bytes, got %zu", need, ws_bytes);
  return launch_route(x, w_r, bias, dt, T, d, E, k, weights, topk_idx, topk_w, logits, ws, stream);
}

int64_t moe_capacity(int64_t T, int32_t k, int32_t E, double factor, int64_t min_capacity) {
  if (T < 0 || k < 1 || E < 1 || !std::isfinite(factor)) return 0;
  constexpr int64_t kMax = (int64_t{1} << 31) - 1;
  const double q = std::ceil(factor * static_cast<double>(T) * static_cast<double>(k) / static_cast<double>(E));
  const int64_t c = q >= static_cast<double>(kMax) ? kMax : (q <= -static_cast<double>(kMax) ? -kMax : static_cast<int64_t>(q));
  const int64_t r = c > min_capacity ? c : min_capacity;
  return r > kMax ? kMax : r;
}

size_t moe_dispatch_workspace_bytes(int64_t T, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || k < 1) return 0;
  return dispatch_ws_bytes(T, E, k);
}

moe_status_t moe_dispatch(const int32_t* topk_idx, const float* logits, int64_t T, int32_t E, int32_t k,
                          int64_t capacity, moe_priority_t priority, moe_overflow_t overflow, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* n_dropped, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  if (T < 0 || T > (int64_t{1} << 31) - 1) return fail(MOE_EINVAL, "T out of range");
  if (E < 1 || E > kMaxExperts) return fail(MOE_EINVAL, "E=%d must be in [1, %d]", E, kMaxExperts);
  if (k < 1 || k > E) return fail(MOE_EINVAL, "k=%d must be in [1, E=%d]", k, E);
  if (T * k > (int64_t{1} << 31) - 1) return fail(MOE_EINVAL, "T*k exceeds 2^31-1");
  if (!counts || !offsets || !n_dropped || !ws || (T > 0 && (!topk_idx || !perm || !inv)))
    return fail(MOE_EINVAL, "moe_dispatch: null required pointer");
  if (priority != MOE_PRIORITY_TOKEN && priority != MOE_PRIORITY_SLOT)
    return fail(MOE_EINVAL, "priority %d invalid", priority);
  if (overflow != MOE_OVERFLOW_DROP && overflow != MOE_OVERFLOW_REROUTE)
    return fail(MOE_EINVAL, "overflow %d invalid", overflow);
  if (capacity > (int64_t{1} << 31) - 1) capacity = 0;   // larger than any count: unlimited
  if (overflow == MOE_OVERFLOW_REROUTE && capacity > 0 && T > 0 && !logits)
    return fail(MOE_EINVAL, "re-routing needs the router logits");
  if (overflow == MOE_OVERFLOW_REROUTE && T * k > (int64_t{1} << 29))
    return fail(MOE_EUNSUPPORTED, "re-routing supports at most 2^29 slots");
  const size_t need = dispatch_ws_bytes(T, E, k);
  if (ws_bytes < need) return fail(MOE_EWORKSPACE, "dispatch needs %zu workspace bytes, got %zu", need, ws_bytes);
  return launch_dispatch(topk_idx, logits, T, E, k, capacity, priority, overflow, counts, offsets, perm, inv,
                         n_dropped, ws, stream);
}

size_t moe_expert_ffn_workspace_bytes(int64_t max_rows, int32_t G, int64_t d, int64_t F, moe_act_t act,
                                      moe_dtype_t dt, const moe_tile_t* tile) {
  if (max_rows < 0 || G < 1 || d < 1 || F < 1) return 0;
  if (check_tile(tile) != MOE_OK) return 0;
  return ffn_plan(max_rows, G, 0, d, F, act, dt, 0, tile_rows_of(tile), tile_waves_of(tile)).ws_bytes;
}

moe_status_t moe_pack_weights(const void* w, void* packed, int64_t G, int64_t N, int64_t K, hipStream_t stream) {
  g_last_error[0] = 0;
  if (G < 1 || N < 1 || K < 1) return fail(MOE_EINVAL, "G, N and K must be >= 1");
  if (N % 16 != 0 || K % 32 != 0)
    return fail(MOE_EUNSUPPORTED, "packing needs N %% 16 == 0 and K %% 32 == 0 (N=%lld K=%lld)", (long long)N,
                (long long)K);
  if (N > (int64_t{1} << 40) / K || G > (int64_t{1} << 60) / (N * K))
    return fail(MOE_EINVAL, "G*N*K too large");
  if (!w || !packed) return fail(MOE_EINVAL, "moe_pack_weights: null pointer");
  if (!aligned16(w) || !aligned16(packed)) return fail(MOE_EINVAL, "w and packed must be 16-byte aligned");
  const uintptr_t bytes = static_cast<uintptr_t>(G * N * K) * 2;
  const uintptr_t a = reinterpret_cast<uintptr_t>(w), b = reinterpret_cast<uintptr_t>(packed);
  if (a < b + bytes && b < a + bytes) return fail(MOE_EINVAL, "w and packed overlap");
  return launch_pack(w, packed, G, N, K, stream);
}

moe_status_t moe_expert_ffn(const void* x, const int32_t* perm, int32_t k, const int32_t* offsets, int32_t G,
                            int64_t max_rows, int64_t d, int64_t F, moe_act_t act, moe_dtype_t dt,
                            moe_layout_t layout, const void* w_gate, const void* w_up, const void* w_down, float* y,
                            const moe_tile_t* tile, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  if (moe_status_t st = check_ffn_args(x, perm, offsets, G, max_rows, d, F, act, dt, w_gate, w_up, w_down, y))
    return st;
  if (moe_status_t st = check_layout(layout, dt)) return st;
  if (moe_status_t st = check_tile(tile)) return st;
  if (perm && k < 1) return fail(MOE_EINVAL, "k must be >= 1 when perm is given");
  const FfnPlan plan = ffn_plan(max_rows, G, 0, d, F, act, dt, 0, tile_rows_of(tile), tile_waves_of(tile));
  if (!ws || ws_bytes < plan.ws_bytes)
    return fail(MOE_EWORKSPACE, "expert FFN needs %zu workspace bytes, got %zu", plan.ws_bytes, ws_bytes);
  FfnProblem p{};
  p.x = x; p.perm = perm; p.k = k; p.offsets = offsets; p.G = G; p.max_rows = max_rows;
  p.d = d; p.F = F; p.act = act; p.dt = dt; p.layout = layout;
  p.w_gate = w_gate; p.w_up = act == MOE_ACT_SWIGLU ? w_up : nullptr; p.w_down = w_down;
  return launch_ffn(p, plan, y, /*reduce_splits=*/true, ws, stream);
}

moe_status_t moe_combine(const float* y, int64_t y_rows, const int32_t* inv, const float* topk_w,
                         const float* shared, int64_t T, int64_t d, int32_t k, moe_dtype_t out_dt, void* out,
                         hipStream_t stream) {
  g_last_error[0] = 0;
  if (!valid_dt(out_dt)) return fail(MOE_EINVAL, "out dtype %d invalid", out_dt);
  if (T < 0 || d < 1 || k < 1 || y_rows < 0) return fail(MOE_EINVAL, "bad sizes (T, d, k, y_rows)");
  if (T > 0 && (!inv || !topk_w || !out || (y_rows > 0 && !y)))
    return fail(MOE_EINVAL, "moe_combine: null required pointer");
  return launch_combine(y, y_rows, 1, 0, inv, topk_w, shared, T, d, k, out_dt, out, stream);
}

size_t moe_routing_stats_workspace_bytes(int64_t T) { return T < 0 ? 0 : stats_ws_bytes(T); }

moe_status_t moe_routing_stats(const float* logits, const int32_t* counts, const int32_t* n_dropped, int64_t T,
                               int32_t E, int32_t k, float lambda_balance, float lambda_aux, float gamma_aux,
                               float* stats, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  if (T < 0 || E < 1 || E > kMaxExperts || k < 1 || k > E) return fail(MOE_EINVAL, "bad sizes (T, E, k)");
  if (T > 0 && (!logits || !counts || !stats || !ws)) return fail(MOE_EINVAL, "moe_routing_stats: null required pointer");
  const size_t need = stats_ws_bytes(T);
  if (ws_bytes < need) return fail(MOE_EWORKSPACE, "routing stats need %zu workspace bytes, got %zu", need, ws_bytes);
  return launch_stats(logits, counts, n_dropped, T, E, k, lambda_balance, lambda_aux, gamma_aux, stats, ws, stream);
}

static size_t layer_layout(const moe_layer_args_t* a, bool carve, WsCarver& c, int32_t** idx, float** w,
                           float** logits, int32_t** counts, int32_t** offsets, int32_t** perm, int32_t** inv,
                           int32_t** ndrop, void** rws, void** sws, void** dws, float** Y, void** fws,
                           FfnPlan* plan) {
  const int64_t T = a->T;
  const bool shared = a->s_gate != nullptr;
  const int64_t max_rows = T * a->k + (shared ? T : 0);
  *plan = ffn_plan(max_rows, a->E, shared ? T : 0, a->d, a->F, a->act, a->dt, a->capacity, a->tile.rows,
                   a->tile.waves);
  float* lg = c.take<float>(static_cast<size_t>(T) * a->E);
  int32_t* ix = c.take<int32_t>(static_cast<size_t>(T) * a->k);
  float* tw = c.take<float>(static_cast<size_t>(T) * a->k);
  int32_t* cn = c.take<int32_t>(a->E);
  int32_t* of = c.take<int32_t>(a->E + 1);
  int32_t* pm = c.take<int32_t>(static_cast<size_t>(T) * a->k);
  int32_t* iv = c.take<int32_t>(static_cast<size_t>(T) * a->k);
  int32_t* nd = c.take<int32_t>(1);
  void* rw = c.take<char>(route_ws_bytes(T, a->d, a->E, a->dt));
  void* sw = c.take<char>(a->stats ? stats_ws_bytes(T) : 0);
  void* dw = c.take<char>(dispatch_ws_bytes(T, a->E, a->k));
  float* yy = c.take<float>(static_cast<size_t>(plan->splits) * max_rows * a->d);
  void* fw = c.take<char>(plan->ws_bytes);
  if (carve) {
    *logits = a->logits ? a->logits : lg;
    *idx = a->topk_idx ? a->topk_idx : ix;
    *w = a->topk_w ? a->topk_w : tw;
    *counts = a->counts ? a->counts : cn;
    *offsets = a->offsets ? a->offsets : of;
    *perm = a->perm ? a->perm : pm;
    *inv = a->inv ? a->inv : iv;
    *ndrop = a->n_dropped ? a->n_dropped : nd;
    *rws = rw;
    *sws = sw;
    *dws = dw;
    *Y = yy;
    *fws = fw;
  }
  return c.off;
}

size_t moe_layer_workspace_bytes(const moe_layer_args_t* a) {
  if (!a || a->T < 0 || a->E < 1 || a->k < 1 || a->d < 1 || a->F < 1) return 0;
  if (check_tile(&a->tile) != MOE_OK) return 0;
  WsCarver c(nullptr);
  int32_t *i, *cn, *of, *pm, *iv, *nd;
  float *w, *lg, *Y;
  void *rws, *sws, *dws, *fws;
  FfnPlan plan;
  return layer_layout(a, false, c, &i, &w, &lg, &cn, &of, &pm, &iv, &nd, &rws, &sws, &dws, &Y, &fws, &plan);
}

// Size, enum and tile checks of the layer arguments (no pointer is examined).
static moe_status_t check_layer_sizes(const moe_layer_args_t* a) {
  if (!valid_dt(a->dt)) return fail(MOE_EINVAL, "dtype %d is not MOE_F32 or MOE_BF16", a->dt);
  if (a->T < 0 || a->T > (int64_t{1} << 31) - 1) return fail(MOE_EINVAL, "T=%lld out of range", (long long)a->T);
  if (a->d < 1) return fail(MOE_EINVAL, "d=%lld must be >= 1", (long long)a->d);
  if (a->E < 1 || a->E > kMaxExperts) return fail(MOE_EINVAL, "E=%d must be in [1, %d]", a->E, kMaxExperts);
  if (a->k < 1 || a->k > a->E) return fail(MOE_EINVAL, "k=%d must be in [1, E=%d]", a->k, a->E);
  if (a->T * a->k > (int64_t{1} << 31) - 1) return fail(MOE_EINVAL, "T*k exceeds 2^31-1");
  if (route_lds_bytes(a->d, a->E, a->dt) > kMaxLdsBytes)
    return fail(MOE_EUNSUPPORTED, "routing %d experts with d=%lld does not fit one workgroup's LDS", a->E,
                (long long)a->d);
  if (!valid_act(a->act)) return fail(MOE_EINVAL, "activation %d invalid", a->act);
  if (a->F < 1) return fail(MOE_EINVAL, "F must be >= 1");
  if (a->dt == MOE_BF16 && (a->d % 64 != 0 || a->F % 64 != 0))
    return fail(MOE_EUNSUPPORTED, "bf16 layer needs d and F multiples of 64");
  if (a->dt == MOE_BF16) {
    if (moe_status_t st = check_bf16_operands(a->T, a->d, a->F)) return st;
  }
  return check_tile(&a->tile);
}

moe_status_t moe_layer_plan(const moe_layer_args_t* a, moe_ffn_plan_t* plan) {
  g_last_error[0] = 0;
  if (!a || !plan) return fail(MOE_EINVAL, "moe_layer_plan: null pointer");
  if (moe_status_t st = check_layer_sizes(a)) return st;
  const bool shared = a->s_gate != nullptr;
  const FfnPlan pl = ffn_plan(a->T * a->k + (shared ? a->T : 0), a->E, shared ? a->T : 0, a->d, a->F, a->act,
                              a->dt, a->capacity, a->tile.rows, a->tile.waves);
  plan->tile_rows = pl.bm;
  plan->tile_waves = a->dt == MOE_BF16 ? pl.nw : 4;
  plan->down_splits = pl.splits;
  return MOE_OK;
}

moe_status_t moe_layer_forward(const moe_layer_args_t* a, hipStream_t stream) {
  g_last_error[0] = 0;
  if (!a) return fail(MOE_EINVAL, "null args");
  if (moe_status_t st = check_route_args(a->x, a->w_r, a->dt, a->T, a->d, a->E, a->k, a->x, a->x, a->x)) return st;
  if (moe_status_t st = check_tile(&a->tile)) return st;
  if (!valid_act(a->act)) return fail(MOE_EINVAL, "activation %d invalid", a->act);
  if (!valid_dt(a->out_dt)) return fail(MOE_EINVAL, "out dtype %d invalid", a->out_dt);
  if (a->weights != MOE_WEIGHTS_RENORMALIZED && a->weights != MOE_WEIGHTS_SOFTMAX)
    return fail(MOE_EINVAL, "weights mode %d invalid", a->weights);
  if (a->priority != MOE_PRIORITY_TOKEN && a->priority != MOE_PRIORITY_SLOT)
    return fail(MOE_EINVAL, "priority %d invalid", a->priority);
  if (a->overflow != MOE_OVERFLOW_DROP && a->overflow != MOE_OVERFLOW_REROUTE)
    return fail(MOE_EINVAL, "overflow %d invalid", a->overflow);
  if (a->overflow == MOE_OVERFLOW_REROUTE && a->T * a->k > (int64_t{1} << 29))
    return fail(MOE_EUNSUPPORTED, "re-routing supports at most 2^29 slots");
  if (moe_status_t st = check_layout(a->layout, a->dt)) return st;
  if (a->F < 1) return fail(MOE_EINVAL, "F must be >= 1");
  if (a->dt == MOE_BF16 && (a->d % 64 != 0 || a->F % 64 != 0))
    return fail(MOE_EUNSUPPORTED, "bf16 layer needs d and F multiples of 64");
  const bool swiglu = a->act == MOE_ACT_SWIGLU;
  if (a->T > 0 && (!a->out || !a->w_gate || !a->w_down || (swiglu && !a->w_up)))
    return fail(MOE_EINVAL, "moe_layer_forward: null required pointer");
  if (a->s_gate && (!a->s_down || (swiglu && !a->s_up)))
    return fail(MOE_EINVAL, "shared expert needs s_gate, s_down (and s_up for SwiGLU)");
  const void* al[] = {a->w_gate, a->w_up, a->w_down, a->s_gate, a->s_up, a->s_down, a->out};
  for (const void* p : al)
    if (p && !aligned16(p)) return fail(MOE_EINVAL, "weights and out must be 16-byte aligned");
  if (a->T == 0) return MOE_OK;
  if (a->dt == MOE_BF16) {
    if (moe_status_t st = check_bf16_operands(a->T, a->d, a->F)) return st;
  }
  const size_t need = moe_layer_workspace_bytes(a);
  if (!a->ws || a->ws_bytes < need)
    return fail(MOE_EWORKSPACE, "layer needs %zu workspace bytes, got %zu", need, a->ws_bytes);
  if (!aligned16(a->ws)) return fail(MOE_EINVAL, "workspace must be 16-byte aligned");

  WsCarver c(a->ws);
  int32_t *idx, *counts, *offsets, *perm, *inv, *ndrop;
  float *w, *logits, *Y;
  void *rws, *sws, *dws, *fws;
  FfnPlan plan;
  layer_layout(a, true, c, &idx, &w, &logits, &counts, &offsets, &perm, &inv, &ndrop, &rws, &sws, &dws, &Y, &fws,
               &plan);

  const int64_t T = a->T;
  const bool shared = a->s_gate != nullptr;
  const int64_t max_rows = T * a->k + (shared ? T : 0);
  int64_t capacity = a->capacity;
  if (capacity > (int64_t{1} << 31) - 1) capacity = 0;

  void* const* ev = a->stage_events;
  auto mark = [&](int i) {
    if (ev) (void)hipEventRecord(static_cast<hipEvent_t>(ev[i]), stream);
  };
  mark(0);
  if (moe_status_t st = launch_route(a->x, a->w_r, a->bias, a->dt, T, a->d, a->E, a->k, a->weights, idx, w, logits,
                                     rws, stream))
    return st;
  mark(1);
  if (moe_status_t st = launch_dispatch(idx, logits, T, a->E, a->k, capacity, a->priority, a->overflow, counts,
                                        offsets, perm, inv, ndrop, dws, stream))
    return st;
  if (a->stats) {
    if (moe_status_t st = launch_stats(logits, counts, ndrop, T, a->E, a->k, a->lambda_balance, a->lambda_aux,
                                       a->gamma_aux, a->stats, sws, stream))
      return st;
  }
  mark(2);
  FfnProblem p{};
  p.x = a->x; p.perm = perm; p.k = a->k; p.offsets = offsets; p.G = a->E; p.max_rows = max_rows;
  p.d = a->d; p.F = a->F; p.act = a->act; p.dt = a->dt; p.layout = a->layout;
  p.w_gate = a->w_gate; p.w_up = swiglu ? a->w_up : nullptr; p.w_down = a->w_down;
  p.s_gate = a->s_gate; p.s_up = swiglu ? a->s_up : nullptr; p.s_down = a->s_down;
  p.shared_rows = shared ? T : 0;
  p.shared_row0 = T * a->k;
  if (moe_status_t st = launch_ffn(p, plan, Y, /*reduce_splits=*/false, fws, stream, ev ? ev + 3 : nullptr))
    return st;
  const float* sh = shared ? Y + T * a->k * a->d : nullptr;
  if (moe_status_t st = launch_combine(Y, T * a->k, plan.splits, max_rows * a->d, inv, w, sh, T, a->d, a->k,
                                       a->out_dt, a->out, stream))
    return st;
  mark(6);
  return MOE_OK;
}

}  // extern "C"
