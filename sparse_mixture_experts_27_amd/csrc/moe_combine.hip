// Combine: out[t] = sum_{kept j} w[t,j] * y[inv[t,j]] (+ shared[t]), fp32 accumulation,
// rounded once to the output dtype.  [200B-5] "谁来决定请哪几个专家？": the selected
// experts' output vectors are mixed by the routing weights (0.75 x E1 + 0.25 x E3);
// "共享专家，给每个token都走的一条路": the shared expert's result is added.
// One workgroup per token, 4-wide vector loads along d; the gathered rows are read in
// full 16-byte pieces, so each expert-output row is streamed once.  If the expert
// outputs are split over K (several partial buffers), the partials are summed first,
// in buffer order, then weighted: the result does not depend on scheduling.
#include "moe_common.h"

namespace moe {
namespace {

template <bool VEC, bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, int64_t y_rows, int nsplit,
                                                      int64_t split_stride, const int32_t* __restrict__ inv,
                                                      const float* __restrict__ topk_w,
                                                      const float* __restrict__ shared, int64_t d, int k,
                                                      void* __restrict__ out) {
  const int64_t t = blockIdx.x;
  constexpr int W = VEC ? 4 : 1;
  for (int64_t c = static_cast<int64_t>(threadIdx.x) * W; c < d; c += 256 * W) {
    float acc[W];
#pragma unroll
    for (int i = 0; i < W; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int32_t r = inv[t * k + j];
      if (r < 0 || r >= y_rows) continue;
      const float w = topk_w[t * k + j];
      float v[W];
      if (VEC) {
        f32x4 q = *reinterpret_cast<const f32x4*>(y + r * d + c);
        for (int s = 1; s < nsplit; ++s) q += *reinterpret_cast<const f32x4*>(y + s * split_stride + r * d + c);
#pragma unroll
        for (int i = 0; i < W; ++i) v[i] = q[i];
      } else {
        v[0] = y[r * d + c];
        for (int s = 1; s < nsplit; ++s) v[0] += y[s * split_stride + r * d + c];
      }
#pragma unroll
      for (int i = 0; i < W; ++i) acc[i] = fmaf(w, v[i], acc[i]);
    }
    if (shared) {
#pragma unroll
      for (int i = 0; i < W; ++i) {
        float sv = shared[t * d + c + i];
        for (int s = 1; s < nsplit; ++s) sv += shared[s * split_stride + t * d + c + i];
        acc[i] += sv;
      }
    }
    if (OUT_BF16) {
      uint16_t* o = static_cast<uint16_t*>(out) + t * d + c;
#pragma unroll
      for (int i = 0; i < W; ++i) o[i] = f32_to_bf16(acc[i]);
    } else {
      float* o = static_cast<float*>(out) + t * d + c;
#pragma unroll
      for (int i = 0; i < W; ++i) o[i] = acc[i];
    }
  }
}

}  // namespace

moe_status_t launch_combine(const float* y, int64_t y_rows, int nsplit, int64_t split_stride,
                            const int32_t* inv, const float* topk_w, const float* shared, int64_t T,
                            int64_t d, int k, int out_dt, void* out, hipStream_t s) {
  if (T == 0) return MOE_OK;
  const bool vec = (d % 4) == 0 && aligned16(y) && (shared == nullptr || aligned16(shared)) &&
                   (split_stride % 4) == 0;
  const unsigned grid = static_cast<unsigned>(T);
  if (out_dt == MOE_BF16) {
    if (vec) combine_kernel<true, true><<<grid, 256, 0, s>>>(y, y_rows, nsplit, split_stride, inv, topk_w, shared, d, k, out);
    else combine_kernel<false, true><<<grid, 256, 0, s>>>(y, y_rows, nsplit, split_stride, inv, topk_w, shared, d, k, out);
  } else {
    if (vec) combine_kernel<true, false><<<grid, 256, 0, s>>>(y, y_rows, nsplit, split_stride, inv, topk_w, shared, d, k, out);
    else combine_kernel<false, false><<<grid, 256, 0, s>>>(y, y_rows, nsplit, split_stride, inv, topk_w, shared, d, k, out);
  }
  return check_launch("combine kernel");
}

}  // namespace moe
