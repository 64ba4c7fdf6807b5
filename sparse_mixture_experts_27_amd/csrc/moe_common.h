// Internal helpers shared by the HIP translation units of libmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <stdarg.h>
#include <stdio.h>

#include "moe.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxExperts = 1024;

// ---- host-side status handling -------------------------------------------------
void set_error(const char* fmt, ...);
moe_status_t fail(moe_status_t s, const char* fmt, ...);
moe_status_t check_launch(const char* what);
// Raise a kernel's dynamic-LDS limit once per (device, kernel).
void set_max_dynamic_smem(const void* func, size_t bytes);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bump allocator over a caller-provided workspace (host arithmetic only).
struct WsCarver {
  char* base;
  size_t off = 0;
  explicit WsCarver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t n) {
    off = align_up(off, 256);
    T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
    off += n * sizeof(T);
    return p;
  }
};

// ---- internal launchers shared between entry points ----------------------------
// The router splits K over workgroups when there are few token blocks; ws holds the
// partial logits (route_ws_bytes; 0 when no split is used).
size_t route_ws_bytes(int64_t T, int64_t d, int E, int dt);
// Dynamic LDS bytes the routing kernels request for these sizes (at most kMaxLdsBytes).
size_t route_lds_bytes(int64_t d, int E, int dt);
constexpr size_t kMaxLdsBytes = 160 * 1024;   // LDS of one gfx950 CU, the most one workgroup can use
moe_status_t launch_route(const void* x, const void* w_r, const float* bias, int dt,
                          int64_t T, int64_t d, int E, int k, int mode, int32_t* topk_idx,
                          float* topk_w, float* logits, void* ws, hipStream_t s);

size_t dispatch_ws_bytes(int64_t T, int E, int k);
moe_status_t launch_dispatch(const int32_t* topk_idx, const float* logits, int64_t T, int E, int k,
                             int64_t capacity, int priority, int overflow, int32_t* counts, int32_t* offsets,
                             int32_t* perm, int32_t* inv, int32_t* n_dropped, void* ws, hipStream_t s);

// One FFN problem: G routed groups (rows from `offsets`, gathered through `perm`)
// plus an optional shared group of `shared_rows` identity rows placed at row
// `shared_row0` of the output.
struct FfnProblem {
  const void* x;
  const int32_t* perm;      // nullable
  int k;                    // divisor for perm entries
  const int32_t* offsets;   // [G+1] device
  int G;
  int64_t max_rows;         // rows of y / H allocated
  int64_t d, F;
  int act, dt;
  int layout;               // moe_layout_t of every expert weight below
  const void* w_gate; const void* w_up; const void* w_down;       // [G, ...]
  const void* s_gate; const void* s_up; const void* s_down;       // shared or null
  int64_t shared_rows;      // 0 = no shared group
  int64_t shared_row0;
};

struct FfnPlan {
  int bm;                   // rows per M-tile
  int nw;                   // waves per workgroup of the bf16 GEMMs (4 or 8)
  int splits;               // split-K factor of the down projection
  int64_t max_mtiles;
  size_t ws_bytes;
};
// shared_rows: rows of the shared group inside max_rows (0 = none); capacity: per-group
// row limit if known (0 = unknown).  Both only tune the tile height.  tile_rows /
// tile_waves: the caller's explicit tile shape (0 = the plan's own choice); a given shape
// must pass bf16_tile_supported.
FfnPlan ffn_plan(int64_t max_rows, int G, int64_t shared_rows, int64_t d, int64_t F, int act, int dt,
                 int64_t capacity, int tile_rows, int tile_waves);
// Whether the bf16 grouped GEMM has a kernel for bm rows per M-tile and nw waves.
bool bf16_tile_supported(int bm, int nw);
// y: [splits][max_rows][d] fp32 partial sums when plan.splits > 1 and reduce_splits is
// false; otherwise [max_rows][d] final.
// ev (nullable): events recorded after the schedule, up-projection and down-projection.
moe_status_t launch_ffn(const FfnProblem& p, const FfnPlan& plan, float* y, bool reduce_splits,
                        void* ws, hipStream_t s, void* const* ev = nullptr);

// Fragment packing of bf16 weights [G, N, K] (moe_pack_weights; sizes already checked).
moe_status_t launch_pack(const void* w, void* packed, int64_t G, int64_t N, int64_t K, hipStream_t s);

size_t stats_ws_bytes(int64_t T);
moe_status_t launch_stats(const float* logits, const int32_t* counts, const int32_t* n_dropped, int64_t T, int E,
                          int k, float lambda_balance, float lambda_aux, float gamma_aux, float* stats, void* ws,
                          hipStream_t s);

moe_status_t launch_combine(const float* y, int64_t y_rows, int nsplit, int64_t split_stride,
                            const int32_t* inv, const float* topk_w, const float* shared,
                            int64_t T, int64_t d, int k, int out_dt, void* out, hipStream_t s);

// ---- device helpers ----------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// fp32 -> bf16, round to nearest even: one v_cvt_pk_bf16_f32 (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

// SiLU v * sigmoid(v) = v / (1 + e^-v), with the hardware exp2 and reciprocal (each within
// about 1 ulp of fp32; the result is rounded to bf16 or feeds an fp32 product): no IEEE
// division sequence in the GEMM epilogues.  Large negative v: e^-v overflows to inf and
// the reciprocal to 0, so the result is -0; large positive v: the reciprocal is 1.
__device__ __forceinline__ float silu_f(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896341f * v));
}
__device__ __forceinline__ float gelu_f(float v) { return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f)); }

}  // namespace moe
