// Routing statistics of one batch: load-balance terms and monitoring metrics.
// [mlqm] www.mlqm.cn/news/130088 §3.1 and §4.2: u_e = fraction of tokens selecting expert
// e, balance ratio std(u)/mean(u) (Bessel's correction), L_balance = lambda * ratio with
// lambda = 0.01.  [cnnet] "MoE混合专家架构原理与工程实践…" §3.2: L_aux = lambda (std(u) +
// gamma max(u)), lambda = 0.01, gamma = 100.  [rkmt] "大模型MoE架构揭秘…" §6.1: per-expert
// utilization ratio, token drop rate, router entropy.
//
// Pass 1 (grid): per-token entropy H_t = ln S - sum_e q_e (z_e - m) / S with m = max z,
// q_e = exp(z_e - m), S = sum_e q_e; one wave per token, fixed butterfly reductions,
// per-block partial sums in double.  Pass 2 (one workgroup): block partials summed in
// block order, counts statistics in double.  Bit-reproducible.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int ST_TOK = 64;   // tokens per block of pass 1 (16 per wave)

__global__ __launch_bounds__(256) void stats_entropy_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                            double* __restrict__ partial) {
  __shared__ double wsum[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double acc = 0.0;
  for (int i = 0; i < ST_TOK / 4; ++i) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * ST_TOK + wave * (ST_TOK / 4) + i;
    if (t >= T) break;                                   // uniform across the wave
    const float* z = logits + t * E;
    float m = -INFINITY;
    for (int e = lane; e < E; e += 64) m = fmaxf(m, z[e]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float s = 0.f, sz = 0.f;
    for (int e = lane; e < E; e += 64) {
      const float d = z[e] - m;
      const float q = expf(d);
      s += q;
      sz += q * d;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      s += __shfl_xor(s, o);
      sz += __shfl_xor(sz, o);
    }
    acc += static_cast<double>(logf(s) - sz / s);
  }
  if (lane == 0) wsum[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
}

// Fixed-order block reduction of one double per thread (1024 threads).
__device__ double block_sum(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int s = 512; s >= 1; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(1024) void stats_final_kernel(const double* __restrict__ partial, int nblocks,
                                                           const int32_t* __restrict__ counts,
                                                           const int32_t* __restrict__ n_dropped, int64_t T, int E,
                                                           int k, float lambda_balance, float lambda_aux,
                                                           float gamma_aux, float* __restrict__ stats) {
  __shared__ double red[1024];
  double ent = 0.0;
  for (int b = threadIdx.x; b < nblocks; b += 1024) ent += partial[b];
  ent = block_sum(ent, red) / static_cast<double>(T);
  const int e = threadIdx.x;                            // E <= 1024
  const double u = e < E ? static_cast<double>(counts[e]) / static_cast<double>(T) : 0.0;
  const double mean = block_sum(u, red) / E;
  const double dev = e < E ? (u - mean) * (u - mean) : 0.0;
  const double var = E > 1 ? block_sum(dev, red) / (E - 1) : 0.0;
  red[threadIdx.x] = e < E ? u : -1.0;
  __syncthreads();
  for (int s = 512; s >= 1; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  const double umax = red[0];
  const double sd = sqrt(var);
  const double slots = static_cast<double>(T) * k;
  if (e < E) stats[5 + e] = static_cast<float>(static_cast<double>(counts[e]) / slots);
  if (threadIdx.x == 0) {
    const double ratio = sd / (mean + 1e-8);
    stats[0] = static_cast<float>(ratio);
    stats[1] = static_cast<float>(lambda_balance * ratio);
    stats[2] = static_cast<float>(lambda_aux * (sd + gamma_aux * umax));
    stats[3] = static_cast<float>(ent);
    stats[4] = static_cast<float>((n_dropped ? static_cast<double>(*n_dropped) : 0.0) / slots);
  }
}

}  // namespace

size_t stats_ws_bytes(int64_t T) {
  return static_cast<size_t>((T + ST_TOK - 1) / ST_TOK) * sizeof(double);
}

moe_status_t launch_stats(const float* logits, const int32_t* counts, const int32_t* n_dropped, int64_t T, int E,
                          int k, float lambda_balance, float lambda_aux, float gamma_aux, float* stats, void* ws,
                          hipStream_t s) {
  if (T == 0) return MOE_OK;
  const int nb = static_cast<int>((T + ST_TOK - 1) / ST_TOK);
  double* partial = static_cast<double*>(ws);
  stats_entropy_kernel<<<nb, 256, 0, s>>>(logits, T, E, partial);
  if (moe_status_t st = check_launch("stats entropy kernel")) return st;
  stats_final_kernel<<<1, 1024, 0, s>>>(partial, nb, counts, n_dropped, T, E, k, lambda_balance, lambda_aux,
                                        gamma_aux, stats);
  return check_launch("stats kernel");
}

}  // namespace moe
