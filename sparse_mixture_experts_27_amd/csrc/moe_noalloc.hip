// moe_layer_forward_noalloc: the layer forward on a fixed, library-owned device scratch
// array instead of a caller workspace, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ variable: every GPU the library runs on holds its
// own copy (MOE_SCRATCH_BYTES) until the process ends.  On the host, `scratch` names a
// host-side stand-in, not a device address, so host code never passes it to a kernel:
// the first call on a device looks up that device's copy with hipGetSymbolAddress (with
// the device current) and keeps the pointer per device; every later use goes through
// that pointer.  The layer's kernels write every scratch word they read within the same
// call (routing buffers, dispatch tables, FFN schedule, hidden activation, expert
// outputs), so nothing needs clearing between calls.  All calls on one GPU share its
// array: calls that overlap in time on one GPU (different streams, or threads without
// ordering) race on it.
#include "moe_common.h"

#include <mutex>

namespace moe {
namespace {

__device__ __align__(256) char scratch[MOE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch` (looked up once per device, the device being current).
moe_status_t device_scratch(void** out) {
  int dev = -1;
  const hipError_t ge = hipGetDevice(&dev);
  if (ge != hipSuccess) return fail(MOE_EHIP, "hipGetDevice: %s", hipGetErrorString(ge));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_EUNSUPPORTED, "device %d: the fixed scratch is kept for devices 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status_t moe_layer_forward_noalloc(const moe_layer_args_t* a, hipStream_t stream) {
  if (!a) return fail(MOE_EINVAL, "null args");
  moe_ffn_plan_t plan;
  if (moe_status_t st = moe_layer_plan(a, &plan)) return st;     // sizes and enums, before any HIP call
  moe_layer_args_t b = *a;
  b.ws = nullptr;
  b.ws_bytes = 0;
  const size_t need = moe_layer_workspace_bytes(&b);
  if (need > MOE_SCRATCH_BYTES)
    return fail(MOE_EWORKSPACE, "this layer call needs %zu bytes of scratch; the fixed scratch holds %zu "
                "(use moe_layer_forward with a workspace, or fewer tokens per call)",
                need, static_cast<size_t>(MOE_SCRATCH_BYTES));
  if (moe_status_t st = device_scratch(&b.ws)) return st;
  b.ws_bytes = MOE_SCRATCH_BYTES;
  return moe_layer_forward(&b, stream);
}
