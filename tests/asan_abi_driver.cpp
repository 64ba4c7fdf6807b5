// Host-side driver for the AddressSanitizer build of the C ABI (tests/test_asan_host.py).
// Every call below is answered on the host - validation failures, pure size and plan
// queries, status strings, error messages - so no GPU is touched.  The driver checks the
// status codes itself and returns non-zero on the first mismatch; AddressSanitizer
// aborts on any invalid host memory access in the library's host code.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <string>
#include <thread>
#include <vector>

#include "moe.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      std::fprintf(stderr, "line %d: %s (last error: %s)\n", __LINE__, #cond, moe_last_error()); \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

// Distinct, 16-byte aligned fake device addresses: validation reads none of them.
static void* fake(uintptr_t i) { return reinterpret_cast<void*>(uintptr_t{1} << 20 | (i << 8)); }

static moe_layer_args_t layer(int64_t T, int32_t E, int32_t k) {
  moe_layer_args_t a;
  std::memset(&a, 0, sizeof(a));
  a.dt = MOE_BF16;
  a.act = MOE_ACT_SWIGLU;
  a.T = T;
  a.d = 4096;
  a.F = 14336;
  a.E = E;
  a.k = k;
  a.x = fake(1);
  a.w_r = fake(2);
  a.w_gate = fake(3);
  a.w_up = fake(4);
  a.w_down = fake(5);
  a.out = fake(6);
  return a;
}

int main() {
  // status strings and the error message buffer
  for (int s = 0; s <= 5; ++s) EXPECT(std::strlen(moe_status_string(static_cast<moe_status_t>(s))) > 0);
  EXPECT(std::strcmp(moe_last_error(), "") == 0);

  // capacity rule: (1024 x 2) / 16 = 128, floor, invalid inputs
  EXPECT(moe_capacity(1024, 2, 16, 1.0, 0) == 128);
  EXPECT(moe_capacity(1, 2, 16, 1.2, 4) == 4);
  EXPECT(moe_capacity(1024, 2, 16, std::nan(""), 4) == 0);
  EXPECT(moe_capacity(-1, 2, 16, 1.0, 0) == 0);
  EXPECT(moe_capacity(int64_t{1} << 40, 1024, 1, 1e300, 0) == (int64_t{1} << 31) - 1);

  // workspace queries
  EXPECT(moe_route_workspace_bytes(16, 4096, 64, MOE_BF16) > 0);
  EXPECT(moe_route_workspace_bytes(-1, 4096, 64, MOE_BF16) == 0);
  EXPECT(moe_dispatch_workspace_bytes(1000, 16, 2) > 0);
  EXPECT(moe_routing_stats_workspace_bytes(-5) == 0);
  const moe_tile_t good{192, 8}, bad{192, 4}, odd{96, 8};
  EXPECT(moe_expert_ffn_workspace_bytes(8192, 64, 4096, 14336, MOE_ACT_SWIGLU, MOE_BF16, &good) > 0);
  EXPECT(moe_expert_ffn_workspace_bytes(8192, 64, 4096, 14336, MOE_ACT_SWIGLU, MOE_BF16, &bad) == 0);
  EXPECT(moe_expert_ffn_workspace_bytes(8192, 64, 4096, 14336, MOE_ACT_SWIGLU, MOE_BF16, &odd) == 0);

  // plans
  moe_layer_args_t a = layer(4096, 64, 2);
  moe_ffn_plan_t plan;
  EXPECT(moe_layer_plan(&a, &plan) == MOE_OK && plan.tile_rows == 192 && plan.tile_waves == 8);
  a.tile = bad;
  EXPECT(moe_layer_plan(&a, &plan) == MOE_EUNSUPPORTED);
  EXPECT(std::strstr(moe_last_error(), "tile") != nullptr);
  a.tile = moe_tile_t{0, 0};
  EXPECT(moe_layer_plan(nullptr, &plan) == MOE_EINVAL);
  EXPECT(moe_layer_plan(&a, nullptr) == MOE_EINVAL);

  // the layer: every rejection happens before a launch
  EXPECT(moe_layer_workspace_bytes(&a) > 0);
  a.ws = fake(7);
  a.ws_bytes = moe_layer_workspace_bytes(&a) - 1;
  EXPECT(moe_layer_forward(&a, nullptr) == MOE_EWORKSPACE);
  a.k = 65;
  EXPECT(moe_layer_forward(&a, nullptr) == MOE_EINVAL);
  a.k = 2;
  a.d = 4000;
  EXPECT(moe_layer_forward(&a, nullptr) == MOE_EUNSUPPORTED);
  a.d = 4096;
  a.T = 300000;                                     // x above 2 GiB
  EXPECT(moe_layer_forward(&a, nullptr) == MOE_EUNSUPPORTED);
  a.T = 0;
  EXPECT(moe_layer_forward(&a, nullptr) == MOE_OK);  // an empty batch launches nothing
  a.T = 4096;
  a.w_up = nullptr;
  EXPECT(moe_layer_forward(&a, nullptr) == MOE_EINVAL);
  a.w_up = fake(4);
  a.layout = 7;
  EXPECT(moe_layer_forward(&a, nullptr) == MOE_EINVAL);
  a.layout = MOE_LAYOUT_LINEAR;
  EXPECT(moe_layer_forward(nullptr, nullptr) == MOE_EINVAL);
  EXPECT(moe_layer_forward_noalloc(&a, nullptr) == MOE_EWORKSPACE);   // prefill-sized: beyond the fixed scratch
  EXPECT(std::strstr(moe_last_error(), "scratch") != nullptr);

  // stage calls
  int32_t* p32 = static_cast<int32_t*>(fake(8));
  float* pf = static_cast<float*>(fake(9));
  EXPECT(moe_route(fake(1), fake(2), nullptr, MOE_BF16, 16, 4096, 64, 65, MOE_WEIGHTS_RENORMALIZED, p32, pf, pf,
                   nullptr, 0, nullptr) == MOE_EINVAL);
  EXPECT(moe_route(fake(1), fake(2), nullptr, MOE_BF16, 16, 4100, 1024, 2, MOE_WEIGHTS_RENORMALIZED, p32, pf, pf,
                   nullptr, 0, nullptr) == MOE_EUNSUPPORTED);
  EXPECT(moe_dispatch(p32, nullptr, 1000, 16, 2, 10, MOE_PRIORITY_TOKEN, MOE_OVERFLOW_REROUTE, p32, p32, p32, p32, p32,
                      fake(10), 1 << 20, nullptr) == MOE_EINVAL);            // re-routing needs the logits
  EXPECT(moe_dispatch(p32, nullptr, 1000, 16, 2, 0, MOE_PRIORITY_TOKEN, MOE_OVERFLOW_DROP, p32, p32, p32, p32, p32,
                      fake(10), 1, nullptr) == MOE_EWORKSPACE);
  EXPECT(moe_expert_ffn(fake(1), p32, 2, p32, 64, 8192, 4096, 14336, MOE_ACT_SWIGLU, MOE_BF16, MOE_LAYOUT_LINEAR,
                        fake(3), fake(4), fake(5), pf, &bad, nullptr, 0, nullptr) == MOE_EUNSUPPORTED);
  EXPECT(moe_expert_ffn(fake(1), nullptr, 1, p32, 64, 300000, 4096, 14336, MOE_ACT_SWIGLU, MOE_BF16,
                        MOE_LAYOUT_LINEAR, fake(3), fake(4), fake(5), pf, nullptr, nullptr, 0, nullptr) == MOE_EUNSUPPORTED);
  EXPECT(moe_combine(pf, 10, p32, pf, nullptr, 4, 64, 2, static_cast<moe_dtype_t>(3), fake(11), nullptr) == MOE_EINVAL);
  EXPECT(moe_routing_stats(pf, p32, p32, 100, 0, 2, 0.01f, 0.01f, 100.f, pf, nullptr, 0, nullptr) == MOE_EINVAL);
  EXPECT(moe_pack_weights(fake(12), static_cast<char*>(fake(12)) + 4096, 2, 32, 64, nullptr) == MOE_EINVAL);  // overlap
  EXPECT(moe_pack_weights(fake(12), fake(13), 2, 24, 64, nullptr) == MOE_EUNSUPPORTED);

  // a long message is truncated to the error buffer, not written past it
  EXPECT(moe_route(nullptr, nullptr, nullptr, static_cast<moe_dtype_t>(9), 1, 1, 1, 1, MOE_WEIGHTS_RENORMALIZED,
                   nullptr, nullptr, nullptr, nullptr, 0, nullptr) == MOE_EINVAL);
  EXPECT(std::strlen(moe_last_error()) < 512);

  // the error message is per host thread
  std::vector<std::thread> ts;
  std::vector<int> ok(8, 0);
  for (int i = 0; i < 8; ++i)
    ts.emplace_back([i, &ok] {
      moe_layer_args_t b = layer(4096, 64, 2);
      b.k = 100 + i;
      for (int r = 0; r < 200; ++r) {
        if (moe_layer_forward(&b, nullptr) != MOE_EINVAL) return;
        if (std::strstr(moe_last_error(), std::to_string(100 + i).c_str()) == nullptr) return;
      }
      ok[i] = 1;
    });
  for (auto& t : ts) t.join();
  for (int i = 0; i < 8; ++i) EXPECT(ok[i] == 1);

  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("asan driver: all checks passed\n");
  return 0;
}
