// Router: logits z = x W_r (+ b), top-k with lowest-index tie-break, renormalised
// weights.  [mlqm] www.mlqm.cn/news/130088 §3.1 (logits = h W_r, softmax, top-k) and
// §3.3 (w_i = p_i / (p_i + p_j)); [200B-5] "谁来决定请哪几个专家？" (top-k).
//
// One workgroup (4 waves) owns 16 tokens.  bf16: the router GEMM runs on
// v_mfma_f32_16x16x32_bf16.  When d is a multiple of 32, a small pass first writes
// W_r transposed to [expert][k] (16 experts padded with zeros) into the workspace, and
// every wave then loads both operands straight from memory in the MFMA layout, wave w
// taking the 32-wide K steps w, w+4, w+8, ...; otherwise W_r is staged through LDS
// transposed, each wave taking a quarter of every 256-wide K chunk.  Either way the
// four partial sums are added in a fixed order, so the logits are bit-reproducible.
// fp32: plain FMA.
// The top-k epilogue runs one 16-lane row per token (the workgroup's 16 tokens at once)
// on a 64-bit key (ordered logit, inverted expert index): the largest key is the largest
// logit, ties going to the lowest index; row maxima and sums use DPP lane moves.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int RT_TOK = 16;     // tokens per workgroup
constexpr int RT_KC = 256;     // K chunk per iteration (4 waves x 64)
constexpr int RT_EB = 64;      // experts per pass of the GEMM
constexpr int RT_PITCH = RT_KC + 8;   // LDS row pitch (elements) of the transposed W_r chunk

// Dynamic LDS layout; the logit rows are sized by E, so E <= 64 stays under 64 KB.
struct RouteSmem {
  uint16_t (*wt)[RT_PITCH];   // [RT_EB][RT_PITCH]  W_r chunk, [expert][k]   (LDS-staged bf16 path)
  float (*red)[RT_TOK][RT_EB];// [4][RT_TOK][RT_EB] per-wave partial logits (bf16 paths)
  float* z;                   // [RT_TOK][E]        final logits of the 16 tokens
  float* zs;                  // [RT_TOK][E]        selected logits, one row per token
  __device__ RouteSmem(char* base, int E, bool wt_buf, bool red_buf) {
    size_t off = 0;
    if (wt_buf) {
      wt = reinterpret_cast<uint16_t(*)[RT_PITCH]>(base);
      off += sizeof(uint16_t) * RT_EB * RT_PITCH;
    }
    if (red_buf) {
      red = reinterpret_cast<float(*)[RT_TOK][RT_EB]>(base + off);
      off += sizeof(float) * 4 * RT_TOK * RT_EB;
    }
    z = reinterpret_cast<float*>(base + off);
    off += sizeof(float) * RT_TOK * E;
    zs = reinterpret_cast<float*>(base + off);
  }
};

inline size_t route_smem_bytes(int E, bool wt_buf, bool red_buf) {
  size_t b = sizeof(float) * (2 * RT_TOK) * static_cast<size_t>(E);
  if (wt_buf) b += sizeof(uint16_t) * RT_EB * RT_PITCH;
  if (red_buf) b += sizeof(float) * 4 * RT_TOK * RT_EB;
  return b;
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const uint16_t v[8]) {
  u32x4 q;
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = static_cast<uint32_t>(v[2 * i]) | (static_cast<uint32_t>(v[2 * i + 1]) << 16);
  return __builtin_bit_cast(bf16x8, q);
}

__device__ __forceinline__ uint32_t ordered_key(float z) {
  uint32_t b = __float_as_uint(z);
  if (b == 0x80000000u) b = 0u;                       // -0 ties with +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t o) {
  uint32_t b = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(b);
}

// Cross-lane steps inside 16-lane rows with DPP (VALU moves, no LDS round trip).
// Controls: quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E, row_ror:4 = 0x124,
// row_ror:8 = 0x128.  After the four steps every lane of a row has combined all 16.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
template <int CTRL>
__device__ __forceinline__ void key_max_step(uint32_t& hi, uint32_t& lo) {
  const uint32_t ohi = dpp_u32<CTRL>(hi), olo = dpp_u32<CTRL>(lo);
  if (ohi > hi || (ohi == hi && olo > lo)) { hi = ohi; lo = olo; }
}
__device__ __forceinline__ void row16_key_max(uint32_t& hi, uint32_t& lo) {
  key_max_step<0xB1>(hi, lo);
  key_max_step<0x4E>(hi, lo);
  key_max_step<0x124>(hi, lo);
  key_max_step<0x128>(hi, lo);
}
// Sum over a 16-lane row in a fixed pattern (the same in every row and every call).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x124>(v);
  v += dpp_f32<0x128>(v);
  return v;
}

// Top-k of one token's logits zrow[0..E) by the 16 lanes of one DPP row (sl = lane % 16
// holds experts sl, sl+16, ...); writes the idx/w rows.  zs: this token's LDS row for the
// selected logits.  Keys are 64-bit (ordered logit, inverted expert index): the largest
// key is the largest logit, ties going to the lowest index.
__device__ void topk_row16(const float* zrow, float* zs, int E, int k, int mode, int32_t* idx_out, float* w_out) {
  const int sl = threadIdx.x & 15;
  const int per_lane = (E + 15) / 16;      // <= 64
  uint64_t removed = 0;
  float z0 = 0.f;
  for (int j = 0; j < k; ++j) {
    uint32_t bhi = 0, blo = 0;             // best remaining candidate of this lane
    for (int i = 0; i < per_lane; ++i) {
      const int e = sl + 16 * i;
      if (e < E && !((removed >> i) & 1u)) {
        const uint32_t hi = ordered_key(zrow[e]);
        const uint32_t lo = 0xffffffffu - static_cast<uint32_t>(e);
        if (hi > bhi || (hi == bhi && lo > blo)) { bhi = hi; blo = lo; }
      }
    }
    row16_key_max(bhi, blo);
    const int e_win = static_cast<int>(0xffffffffu - blo);
    if ((e_win & 15) == sl) removed |= uint64_t{1} << (e_win >> 4);
    const float zw = key_to_float(bhi);
    if (j == 0) z0 = zw;
    if (sl == 0) { idx_out[j] = e_win; zs[j] = zw; }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  // renormalised: w_j = exp(z_j - z_0) / sum_{i<k} exp(z_i - z_0)
  // softmax mode:  w_j = exp(z_j - z_0) / sum_{all e} exp(z_e - z_0)   (z_0 is the max)
  float part = 0.f;
  if (mode == MOE_WEIGHTS_SOFTMAX) {
    for (int e = sl; e < E; e += 16) part += expf(zrow[e] - z0);
  } else {
    for (int j = sl; j < k; j += 16) part += expf(zs[j] - z0);
  }
  const float inv = 1.0f / row16_sum(part);
  for (int j = sl; j < k; j += 16) w_out[j] = expf(zs[j] - z0) * inv;
  __builtin_amdgcn_wave_barrier();
}

// The workgroup's 16 tokens, one per 16-lane row (wave w: tokens 4w..4w+3).
__device__ void finish_tokens(RouteSmem& sm, int64_t tok0, int64_t T, int E, int k, int mode,
                              int32_t* topk_idx, float* topk_w) {
  const int t = threadIdx.x >> 4;
  const int64_t tok = tok0 + t;
  if (tok < T) topk_row16(sm.z + t * E, sm.zs + t * k, E, k, mode, topk_idx + tok * k, topk_w + tok * k);
}

// blockIdx.y selects a K range [ky*kchunk, (ky+1)*kchunk).  With one range the kernel
// finishes the tokens (bias, logits, top-k); with several it writes its partial logits to
// partial[ky][t][e] and route_finish_kernel adds the ranges in index order.
__global__ __launch_bounds__(256) void route_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_r, const float* __restrict__ bias,
    int64_t T, int64_t d, int E, int k, int mode, int64_t kchunk, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ logits, float* __restrict__ partial) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  RouteSmem sm(smem_raw, E, true, true);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * RT_TOK;
  const bool split = gridDim.y > 1;
  const int64_t kb = static_cast<int64_t>(blockIdx.y) * kchunk;
  const int64_t ke = kb + kchunk < d ? kb + kchunk : d;
  const int64_t my_tok = tok0 + (lane & 15);
  const bool tok_ok = my_tok < T;
  const uint16_t* xrow = x + (tok_ok ? my_tok : 0) * d;
  const bool vec_w = (E % 8) == 0;
  const bool vec_x = (d % 8) == 0;

  for (int e0 = 0; e0 < E; e0 += RT_EB) {
    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t k0 = kb; k0 < ke; k0 += RT_KC) {
      __syncthreads();   // previous chunk fully consumed
      // stage W_r[k0 : k0+256, e0 : e0+64] transposed into sm.wt[e][k]
      for (int p = 0; p < RT_KC / 32; ++p) {
        const int row = p * 32 + (tid >> 3);
        const int ec = (tid & 7) * 8;
        const int64_t kk = k0 + row;
        uint16_t v[8];
        if (vec_w && kk < ke && e0 + ec + 8 <= E) {
          const u32x4 q = *reinterpret_cast<const u32x4*>(w_r + kk * E + e0 + ec);
#pragma unroll
          for (int i = 0; i < 4; ++i) { v[2 * i] = q[i] & 0xffff; v[2 * i + 1] = q[i] >> 16; }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            v[i] = (kk < ke && e0 + ec + i < E) ? w_r[kk * E + e0 + ec + i] : 0;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) sm.wt[ec + i][row] = v[i];
      }
      __syncthreads();
      // wave w: k range [k0 + 64w, k0 + 64w + 64) as two 32-deep MFMA steps
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int kl = wave * 64 + s * 32;
        const int64_t kx = k0 + kl + 8 * (lane >> 4);
        bf16x8 a;
        if (tok_ok && vec_x && k0 + kl + 32 <= ke) {
          a = *reinterpret_cast<const bf16x8*>(xrow + kx);
        } else {
          uint16_t v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = (tok_ok && kx + i < ke) ? xrow[kx + i] : 0;
          a = pack_bf16x8(v);
        }
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) {
          if (e0 + nf * 16 < E) {
            const bf16x8 b = *reinterpret_cast<const bf16x8*>(&sm.wt[nf * 16 + (lane & 15)][kl + 8 * (lane >> 4)]);
            acc[nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[nf], 0, 0, 0);
          }
        }
      }
    }
    // C layout of the 16x16 MFMA: lane holds rows 4*(lane/16)+v, column lane%16
#pragma unroll
    for (int nf = 0; nf < 4; ++nf)
#pragma unroll
      for (int v = 0; v < 4; ++v) sm.red[wave][4 * (lane >> 4) + v][nf * 16 + (lane & 15)] = acc[nf][v];
    __syncthreads();
    for (int i = tid; i < RT_TOK * RT_EB; i += 256) {
      const int t = i / RT_EB, e = e0 + i % RT_EB;
      if (e < E) {
        float z = ((sm.red[0][t][i % RT_EB] + sm.red[1][t][i % RT_EB]) + sm.red[2][t][i % RT_EB]) +
                  sm.red[3][t][i % RT_EB];
        if (split) {
          if (tok0 + t < T) partial[(static_cast<int64_t>(blockIdx.y) * T + tok0 + t) * E + e] = z;
        } else {
          if (bias) z += bias[e];
          sm.z[t * E + e] = z;
          if (tok0 + t < T) logits[(tok0 + t) * E + e] = z;
        }
      }
    }
  }
  if (split) return;
  __syncthreads();
  finish_tokens(sm, tok0, T, E, k, mode, topk_idx, topk_w);
}

// W_r [d, E] -> wt [Ep, d] (Ep = E rounded up to 16, padding rows zero); 32 k x 64 e
// tiles, 4-byte accesses on both sides.  d % 32 == 0 here; E may be odd.
__global__ __launch_bounds__(256) void route_transpose_kernel(const uint16_t* __restrict__ w_r, int64_t d, int E,
                                                              int Ep, uint16_t* __restrict__ wt) {
  __shared__ uint16_t tile[32][66];
  const int64_t k0 = static_cast<int64_t>(blockIdx.x) * 32;
  const int e0 = blockIdx.y * 64;
  const int t = threadIdx.x;
  {                                                  // read: row kk, experts 2q, 2q+1
    const int kk = t >> 3, q0 = (t & 7) * 4;
    const uint16_t* row = w_r + (k0 + kk) * E;
#pragma unroll
    for (int q = q0; q < q0 + 4; ++q) {
      const int e = e0 + 2 * q;
      uint32_t w;
      if ((E & 1) == 0)                              // pairs are 4-byte aligned
        w = e < E ? *reinterpret_cast<const uint32_t*>(row + e) : 0u;
      else
        w = (e < E ? row[e] : 0u) | ((e + 1 < E ? static_cast<uint32_t>(row[e + 1]) : 0u) << 16);
      tile[kk][2 * q] = static_cast<uint16_t>(w & 0xffff);
      tile[kk][2 * q + 1] = static_cast<uint16_t>(w >> 16);
    }
  }
  __syncthreads();
  {                                                  // write: expert row ee, k pairs
    const int ee = t >> 2, kq = (t & 3) * 8;
    if (e0 + ee < Ep) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(wt + static_cast<int64_t>(e0 + ee) * d + k0 + kq);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dst[j] = static_cast<uint32_t>(tile[kq + 2 * j][ee]) | (static_cast<uint32_t>(tile[kq + 2 * j + 1][ee]) << 16);
    }
  }
}

// Router GEMM with both operands loaded from memory in the MFMA layout (d % 32 == 0):
// A = 16 token rows of x, B = 16-expert row blocks of wt [Ep, d].  blockIdx.y selects a
// K range as in route_bf16_kernel; within it wave w takes the K steps w, w+4, ...
__global__ __launch_bounds__(256) void route_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wt, const float* __restrict__ bias,
    int64_t T, int64_t d, int E, int Ep, int k, int mode, int64_t kchunk, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ logits, float* __restrict__ partial) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  RouteSmem sm(smem_raw, E, false, true);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * RT_TOK;
  const bool split = gridDim.y > 1;
  const int64_t kb = static_cast<int64_t>(blockIdx.y) * kchunk;
  const int64_t ke = kb + kchunk < d ? kb + kchunk : d;
  const int nsteps = ke > kb ? static_cast<int>((ke - kb) / 32) : 0;
  const int64_t my_tok = tok0 + (lane & 15);
  const uint16_t* xrow = x + (my_tok < T ? my_tok : 0) * d + kb + 8 * (lane >> 4);   // rows past T: ignored
  constexpr int U = 4;                       // K steps in flight per wave

  for (int e0 = 0; e0 < Ep; e0 += RT_EB) {
    const int nfr = (Ep - e0) / 16 < 4 ? (Ep - e0) / 16 : 4;   // 16-expert blocks in this pass
    const uint16_t* wrow = wt + static_cast<int64_t>(e0 + (lane & 15)) * d + kb + 8 * (lane >> 4);
    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Batches of U K steps, double-buffered: the next batch's loads are issued before the
    // current batch's MFMAs, so one memory latency covers the whole walk rather than one
    // per batch.
    bf16x8 a[2][U], b[2][U][4];
    auto load = [&](int buf, int j0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + 4 * u < nsteps ? j0 + 4 * u : j0;    // past the range: a repeated step, not used
        a[buf][u] = *reinterpret_cast<const bf16x8*>(xrow + j * 32);
#pragma unroll
        for (int nf = 0; nf < 4; ++nf)
          b[buf][u][nf] =
              *reinterpret_cast<const bf16x8*>(wrow + static_cast<int64_t>(nf < nfr ? nf : 0) * 16 * d + j * 32);
      }
    };
    auto mul = [&](int buf, int j0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (j0 + 4 * u < nsteps) {
#pragma unroll
          for (int nf = 0; nf < 4; ++nf)
            if (nf < nfr) acc[nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[buf][u], b[buf][u][nf], acc[nf], 0, 0, 0);
        }
      }
    };
    int j0 = wave;
    if (j0 < nsteps) load(0, j0);
    while (j0 < nsteps) {
      int jn = j0 + 4 * U;
      if (jn < nsteps) load(1, jn);
      mul(0, j0);
      j0 = jn;
      if (j0 >= nsteps) break;
      jn = j0 + 4 * U;
      if (jn < nsteps) load(0, jn);
      mul(1, j0);
      j0 = jn;
    }
    // C layout of the 16x16 MFMA: lane holds rows 4*(lane/16)+v, column lane%16
    __syncthreads();                         // previous pass's partials consumed
#pragma unroll
    for (int nf = 0; nf < 4; ++nf)
#pragma unroll
      for (int v = 0; v < 4; ++v) sm.red[wave][4 * (lane >> 4) + v][nf * 16 + (lane & 15)] = acc[nf][v];
    __syncthreads();
    for (int i = tid; i < RT_TOK * RT_EB; i += 256) {
      const int t = i / RT_EB, e = e0 + i % RT_EB;
      if (e < E) {
        float z = ((sm.red[0][t][i % RT_EB] + sm.red[1][t][i % RT_EB]) + sm.red[2][t][i % RT_EB]) +
                  sm.red[3][t][i % RT_EB];
        if (split) {
          if (tok0 + t < T) partial[(static_cast<int64_t>(blockIdx.y) * T + tok0 + t) * E + e] = z;
        } else {
          if (bias) z += bias[e];
          sm.z[t * E + e] = z;
          if (tok0 + t < T) logits[(tok0 + t) * E + e] = z;
        }
      }
    }
  }
  if (split) return;
  __syncthreads();
  finish_tokens(sm, tok0, T, E, k, mode, topk_idx, topk_w);
}

// Sum the K-range partial logits in range order, add the offsets, finish the tokens.
__global__ __launch_bounds__(256) void route_finish_kernel(const float* __restrict__ partial, int nsplit,
                                                           const float* __restrict__ bias, int64_t T, int E,
                                                           int k, int mode, int32_t* __restrict__ topk_idx,
                                                           float* __restrict__ topk_w, float* __restrict__ logits) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  RouteSmem sm(smem_raw, E, false, false);
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * RT_TOK;
  for (int i = threadIdx.x; i < RT_TOK * E; i += 256) {
    const int t = i / E, e = i % E;
    const int64_t tok = tok0 + t;
    float z = 0.f;
    if (tok < T) {
      // issue the loads of up to 16 ranges before the (ordered) additions
      for (int s0 = 0; s0 < nsplit; s0 += 16) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          v[j] = s0 + j < nsplit ? partial[(static_cast<int64_t>(s0 + j) * T + tok) * E + e] : 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (s0 + j < nsplit) z = (s0 + j == 0) ? v[j] : z + v[j];
      }
      if (bias) z += bias[e];
      logits[tok * E + e] = z;
    }
    sm.z[t * E + e] = z;
  }
  __syncthreads();
  finish_tokens(sm, tok0, T, E, k, mode, topk_idx, topk_w);
}

__global__ __launch_bounds__(256) void route_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ w_r, const float* __restrict__ bias,
    int64_t T, int64_t d, int E, int k, int mode, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  RouteSmem sm(smem_raw, E, false, false);
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * RT_TOK;
  for (int i = threadIdx.x; i < RT_TOK * E; i += 256) {
    const int t = i / E, e = i % E;
    const int64_t tok = tok0 + t;
    float z = 0.f;
    if (tok < T) {
      const float* xr = x + tok * d;
      for (int64_t c = 0; c < d; ++c) z = fmaf(xr[c], w_r[c * E + e], z);
      if (bias) z += bias[e];
      logits[tok * E + e] = z;
    }
    sm.z[t * E + e] = z;
  }
  __syncthreads();
  finish_tokens(sm, tok0, T, E, k, mode, topk_idx, topk_w);
}

}  // namespace

int route_splits(int64_t T, int64_t d, int dt) {
  if (dt != MOE_BF16) return 1;
  const int64_t blocks = (T + RT_TOK - 1) / RT_TOK;
  const int64_t chunks = (d + RT_KC - 1) / RT_KC;
  int ks = 1;
  while (blocks * ks < 256 && chunks >= 2 * ks) ks *= 2;
  return ks;
}

// The transposed-operand router needs d % 32 == 0 (whole 32-wide K steps in every range).
bool route_direct(int64_t d, int dt) { return dt == MOE_BF16 && d % 32 == 0; }
int route_padded_experts(int E) { return (E + 15) / 16 * 16; }

size_t route_wt_bytes(int64_t d, int E, int dt) {
  return route_direct(d, dt) ? align_up(static_cast<size_t>(route_padded_experts(E)) * d * sizeof(uint16_t), 256) : 0;
}

size_t route_lds_bytes(int64_t d, int E, int dt) {
  // the largest dynamic LDS request of the routing kernels for these sizes
  if (dt != MOE_BF16) return route_smem_bytes(E, false, false);
  return route_smem_bytes(E, !route_direct(d, dt), true);
}

size_t route_ws_bytes(int64_t T, int64_t d, int E, int dt) {
  const int ks = route_splits(T, d, dt);
  return route_wt_bytes(d, E, dt) + (ks > 1 ? static_cast<size_t>(ks) * T * E * sizeof(float) : 0);
}

moe_status_t launch_route(const void* x, const void* w_r, const float* bias, int dt, int64_t T,
                          int64_t d, int E, int k, int mode, int32_t* topk_idx, float* topk_w, float* logits,
                          void* ws, hipStream_t s) {
  if (T == 0) return MOE_OK;
  const unsigned grid = static_cast<unsigned>((T + RT_TOK - 1) / RT_TOK);
  if (dt == MOE_BF16) {
    const int ks = route_splits(T, d, dt);
    const int64_t chunks = (d + RT_KC - 1) / RT_KC;
    const int64_t kchunk = ((chunks + ks - 1) / ks) * RT_KC;
    const size_t smem = route_smem_bytes(E, !route_direct(d, dt), true);
    const size_t wtb = route_wt_bytes(d, E, dt);
    float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + wtb);
    if (route_direct(d, dt)) {
      const int Ep = route_padded_experts(E);
      uint16_t* wt = static_cast<uint16_t*>(ws);
      route_transpose_kernel<<<dim3(static_cast<unsigned>(d / 32), static_cast<unsigned>((Ep + 63) / 64)), 256,
                               0, s>>>(static_cast<const uint16_t*>(w_r), d, E, Ep, wt);
      if (moe_status_t st = check_launch("route transpose kernel")) return st;
      set_max_dynamic_smem(reinterpret_cast<const void*>(route_mfma_kernel), smem);
      route_mfma_kernel<<<dim3(grid, ks), 256, smem, s>>>(static_cast<const uint16_t*>(x), wt, bias, T, d, E, Ep, k,
                                                          mode, kchunk, topk_idx, topk_w, logits, partial);
    } else {
      set_max_dynamic_smem(reinterpret_cast<const void*>(route_bf16_kernel), smem);
      route_bf16_kernel<<<dim3(grid, ks), 256, smem, s>>>(static_cast<const uint16_t*>(x),
                                                          static_cast<const uint16_t*>(w_r), bias, T, d, E, k,
                                                          mode, kchunk, topk_idx, topk_w, logits, partial);
    }
    if (moe_status_t st = check_launch("route kernel")) return st;
    if (ks > 1) {
      const size_t smem2 = route_smem_bytes(E, false, false);
      set_max_dynamic_smem(reinterpret_cast<const void*>(route_finish_kernel), smem2);
      route_finish_kernel<<<grid, 256, smem2, s>>>(partial, ks, bias, T, E, k, mode, topk_idx, topk_w, logits);
      return check_launch("route finish kernel");
    }
    return MOE_OK;
  }
  const size_t smem = route_smem_bytes(E, false, false);
  set_max_dynamic_smem(reinterpret_cast<const void*>(route_f32_kernel), smem);
  route_f32_kernel<<<grid, 256, smem, s>>>(static_cast<const float*>(x), static_cast<const float*>(w_r), bias, T,
                                           d, E, k, mode, topk_idx, topk_w, logits);
  return check_launch("route kernel");
}

}  // namespace moe
