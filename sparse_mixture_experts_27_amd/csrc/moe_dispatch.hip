// Dispatch: per-expert counts, capacity, expert-sorted permutation.
// [rkmt] "大模型MoE架构揭秘：为什么总参数≠激活参数" §2.3: each expert takes at most C
// slots, the overflow is dropped; [200B-5] "四个专家同时算，选两个会更快吗？": every
// selection is one call of one expert.  The kept slots of one expert are the earliest
// tokens, laid out in ascending token order (a stable counting sort by expert).
//
// Three integer-only passes, bit-deterministic:
//   1. count:   per block of 256 tokens, LDS histogram -> block_counts[b][e]
//   2. scan:    per expert, exclusive scan over blocks -> block_base[b][e]; counts,
//               kept = min(counts, C), offsets = exclusive scan of kept, n_dropped
//   3. scatter: rank of each slot inside its expert = block_base + earlier waves of
//               the block + earlier lanes of the wave; kept slots go to
//               perm[offsets[e] + rank], inv gets the row or -1
// A batch of at most 256 tokens runs all three in one workgroup.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int DP_TOK = 256;   // tokens per block (4 waves x 64 lanes, one token per lane)

__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ idx,
                                                             int64_t T, int E, int k,
                                                             int32_t* __restrict__ block_counts) {
  __shared__ int32_t cnt[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * DP_TOK + threadIdx.x;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int32_t e = idx[t * k + j];
      if (static_cast<uint32_t>(e) < static_cast<uint32_t>(E)) atomicAdd(&cnt[e], 1);
    }
  __syncthreads();
  int32_t* out = block_counts + static_cast<int64_t>(blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += 256) out[e] = cnt[e];
}

// Single workgroup of 1024 threads; thread e owns expert e.
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(const int32_t* __restrict__ block_counts,
                                                             int nblocks, int E, int64_t capacity,
                                                             int32_t* __restrict__ block_base,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ n_dropped) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t wdrop[16];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  int32_t total = 0;
  if (e < E) {
    for (int b = 0; b < nblocks; ++b) {
      block_base[static_cast<int64_t>(b) * E + e] = total;
      total += block_counts[static_cast<int64_t>(b) * E + e];
    }
    counts[e] = total;
  }
  const int32_t kept = (e < E) ? (capacity > 0 && total > capacity ? static_cast<int32_t>(capacity) : total) : 0;
  int32_t drop = (e < E) ? total - kept : 0;
  // inclusive scan of kept across the workgroup (wave scan + wave totals)
  int32_t v = kept;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) drop += __shfl_xor(drop, off);
  if (lane == 63) wsum[wave] = v;
  if (lane == 0) wdrop[wave] = drop;
  __syncthreads();
  int32_t before = 0, dsum = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) before += wsum[w];
    dsum += wdrop[w];
  }
  const int32_t incl = before + v;
  if (e < E) offsets[e + 1] = incl;
  if (e == 0) { offsets[0] = 0; *n_dropped = dsum; }
}

// Place the slots of one block of 256 tokens (one token per thread).  wcnt[w][e] must
// hold the per-wave demand of this block; block_base(e) is the number of earlier tokens
// (in earlier blocks) that chose e, offsets[e] the first row of e.
template <typename BaseFn>
__device__ void scatter_block(const int32_t* __restrict__ idx, int64_t T, int E, int k, int64_t capacity,
                              BaseFn block_base, const int32_t* offsets, int32_t (*wcnt)[kMaxExperts],
                              int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * DP_TOK + threadIdx.x;
  const bool valid = t < T;
  for (int j = 0; j < k; ++j) {
    int32_t e = valid ? idx[t * k + j] : -1;
    if (static_cast<uint32_t>(e) >= static_cast<uint32_t>(E)) e = -1;   // ignored slot
    // lanes below me (earlier tokens of this wave) that selected e in any slot; a
    // token never selects one expert twice
    int32_t rank = 0;
    for (int j2 = 0; j2 < k; ++j2) {
      const int32_t v = valid ? idx[t * k + j2] : -2;
      for (int src = 0; src < 64; ++src) {
        const int32_t es = __shfl(v, src);
        rank += (src < lane && es == e) ? 1 : 0;
      }
    }
    if (valid && e < 0) inv[t * k + j] = -1;
    if (e >= 0) {
      int32_t r = block_base(e) + rank;
      for (int w = 0; w < wave; ++w) r += wcnt[w][e];
      const int64_t slot = t * k + j;
      if (capacity > 0 && r >= capacity) {
        inv[slot] = -1;
      } else {
        const int32_t row = offsets[e] + r;
        perm[row] = static_cast<int32_t>(slot);
        inv[slot] = row;
      }
    }
  }
}

// Per-wave demand of this block into wcnt (zeroed here).
__device__ void count_block(const int32_t* __restrict__ idx, int64_t T, int E, int k,
                            int32_t (*wcnt)[kMaxExperts]) {
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * E; i += 256) wcnt[i / E][i % E] = 0;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * DP_TOK + threadIdx.x;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int32_t e = idx[t * k + j];
      if (static_cast<uint32_t>(e) < static_cast<uint32_t>(E)) atomicAdd(&wcnt[wave][e], 1);
    }
  __syncthreads();
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t T, int E, int k, int64_t capacity,
    const int32_t* __restrict__ block_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int32_t wcnt[4][kMaxExperts];
  count_block(idx, T, E, k, wcnt);
  const int32_t* bb = block_base + static_cast<int64_t>(blockIdx.x) * E;
  scatter_block(idx, T, E, k, capacity, [&](int e) { return bb[e]; }, offsets, wcnt, perm, inv);
}

// All of dispatch in one workgroup when the batch fits one block (T <= 256): demand,
// kept counts, offsets and drops are computed in LDS, then the slots are placed.
__global__ __launch_bounds__(256) void dispatch_small_kernel(
    const int32_t* __restrict__ idx, int64_t T, int E, int k, int64_t capacity,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, int32_t* __restrict__ n_dropped) {
  __shared__ int32_t wcnt[4][kMaxExperts];
  __shared__ int32_t off[kMaxExperts + 1];
  __shared__ int32_t wsum[4], wdrop[4];
  count_block(idx, T, E, k, wcnt);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // thread i owns experts 4i .. 4i+3 (E <= 1024)
  int32_t kept_loc[4];
  int32_t sum = 0, drop = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = threadIdx.x * 4 + q;
    int32_t c = 0, kept = 0;
    if (e < E) {
      c = wcnt[0][e] + wcnt[1][e] + wcnt[2][e] + wcnt[3][e];
      kept = (capacity > 0 && c > capacity) ? static_cast<int32_t>(capacity) : c;
      counts[e] = c;
    }
    kept_loc[q] = kept;
    sum += kept;
    drop += c - kept;
  }
  int32_t v = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t x = __shfl_up(v, o);
    if (lane >= o) v += x;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) drop += __shfl_xor(drop, o);
  if (lane == 63) wsum[wave] = v;
  if (lane == 0) wdrop[wave] = drop;
  __syncthreads();
  int32_t before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  int32_t run = before + v - sum;               // exclusive prefix of this thread's first expert
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = threadIdx.x * 4 + q;
    if (e < E) {
      off[e] = run;
      offsets[e] = run;
    }
    run += kept_loc[q];
  }
  if (threadIdx.x == 0) {
    const int32_t total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    off[E] = total;
    offsets[E] = total;
    *n_dropped = wdrop[0] + wdrop[1] + wdrop[2] + wdrop[3];
  }
  __syncthreads();
  scatter_block(idx, T, E, k, capacity, [](int) { return 0; }, off, wcnt, perm, inv);
}

}  // namespace

size_t dispatch_ws_bytes(int64_t T, int E) {
  const int64_t nb = (T + DP_TOK - 1) / DP_TOK;
  return 2 * align_up(static_cast<size_t>(nb) * E * sizeof(int32_t), 256);
}

moe_status_t launch_dispatch(const int32_t* topk_idx, int64_t T, int E, int k, int64_t capacity,
                             int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                             int32_t* n_dropped, void* ws, hipStream_t s) {
  const int64_t nb = (T + DP_TOK - 1) / DP_TOK;
  WsCarver c(ws);
  int32_t* block_counts = c.take<int32_t>(static_cast<size_t>(nb) * E);
  int32_t* block_base = c.take<int32_t>(static_cast<size_t>(nb) * E);
  if (nb <= 1) {
    const int64_t Tg = nb == 0 ? 0 : T;
    dispatch_small_kernel<<<1, 256, 0, s>>>(topk_idx, Tg, E, k, capacity, counts, offsets, perm, inv, n_dropped);
    return check_launch("dispatch kernel");
  }
  dispatch_count_kernel<<<static_cast<unsigned>(nb), 256, 0, s>>>(topk_idx, T, E, k, block_counts);
  if (moe_status_t st = check_launch("dispatch count kernel")) return st;
  dispatch_scan_kernel<<<1, 1024, 0, s>>>(block_counts, static_cast<int>(nb), E, capacity, block_base,
                                          counts, offsets, n_dropped);
  if (moe_status_t st = check_launch("dispatch scan kernel")) return st;
  dispatch_scatter_kernel<<<static_cast<unsigned>(nb), 256, 0, s>>>(topk_idx, T, E, k, capacity,
                                                                    block_base, offsets, perm, inv);
  if (moe_status_t st = check_launch("dispatch scatter kernel")) return st;
  return MOE_OK;
}

}  // namespace moe
