// Host-only driver of the C ABI's host code (k3moe_api.cpp argument validation and workspace
// layout, expert_cache.cpp), built by tests/test_host_sanitize.py with the host side under
// AddressSanitizer and UndefinedBehaviorSanitizer. Every call here either fails validation
// or needs no GPU (T = 0, sizing, the slot plan, release with nothing created), so no HIP
// call is ever made and no device is needed.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "k3moe.h"

static int fails = 0;
#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++fails;                                                          \
    }                                                                   \
  } while (0)

static bool has_msg() { return k3moe_last_error() && std::strlen(k3moe_last_error()) > 0; }

int main() {
  // never dereferenced: every call below fails validation before any device access
  void* const F = reinterpret_cast<void*>(uintptr_t(0x100000));
  void* const F_odd = reinterpret_cast<void*>(uintptr_t(0x100008));
  const auto* Fu8 = static_cast<const uint8_t*>(F);
  const auto* Fu16 = static_cast<const uint16_t*>(F);
  k3moe_dims K3{7168, 1536, 896, 16};
  k3moe_mx_experts ex{Fu8, Fu8, Fu8, Fu8, Fu8, Fu8};
  const size_t big = size_t(1) << 40;

  CHECK(k3moe_version() == K3MOE_VERSION);
  CHECK(k3moe_release() == K3MOE_OK);  // nothing created yet
  CHECK(k3moe_time_next_kernel(99, nullptr, nullptr) == K3MOE_EINVAL && has_msg());
  CHECK(k3moe_time_next_kernel(K3MOE_KERNEL_DOWN, nullptr, nullptr) == K3MOE_OK);

  // workspace sizes: zero for invalid dims, monotone in T for valid ones
  const k3moe_dims shapes[] = {{7168, 1536, 896, 16}, {512, 256, 32, 4}, {96, 64, 13, 3},
                               {64, 32, 1, 1},        {160, 96, 5, 5},  {16384, 16384, 4096, 32}};
  for (const auto& dm : shapes) {
    size_t prev = 0;
    for (int T : {0, 1, 2, 9, 10, 15, 16, 31, 32, 63, 64, 65, 100, 1000, 2048, 8192}) {
      const size_t n = k3moe_workspace_bytes(&dm, T);
      CHECK(n > 0 && n >= prev);
      prev = n;
    }
  }
  const k3moe_dims bad[] = {{33, 1536, 896, 16}, {7168, 40, 896, 16}, {7168, 1536, 0, 1},
                            {7168, 1536, 896, 0}, {7168, 1536, 8, 9},  {7168, 1536, 896, 33},
                            {32768, 1536, 896, 16}, {7168, 1536, 5000, 16}};
  for (const auto& dm : bad) CHECK(k3moe_workspace_bytes(&dm, 1) == 0);
  CHECK(k3moe_workspace_bytes(nullptr, 1) == 0);
  CHECK(k3moe_workspace_bytes(&K3, -1) == 0);

  int32_t* ids = static_cast<int32_t*>(F);
  float* gates = static_cast<float*>(F);
  float* y = static_cast<float*>(F);
  // router
  CHECK(k3moe_router(nullptr, 1, F, 0, Fu16, nullptr, ids, gates, F, big, nullptr) ==
        K3MOE_EINVAL && has_msg());
  for (const auto& dm : bad)
    CHECK(k3moe_router(&dm, 1, F, 0, Fu16, nullptr, ids, gates, F, big, nullptr) < 0);
  CHECK(k3moe_router(&K3, -1, F, 0, Fu16, nullptr, ids, gates, F, big, nullptr) == K3MOE_EINVAL);
  CHECK(k3moe_router(&K3, 0, F, 0, Fu16, nullptr, ids, gates, F, big, nullptr) == K3MOE_OK);
  CHECK(k3moe_router(&K3, (1 << 20) + 1, F, 0, Fu16, nullptr, ids, gates, F, big, nullptr) ==
        K3MOE_EUNSUPPORTED);
  CHECK(k3moe_router(&K3, 1, F, 7, Fu16, nullptr, ids, gates, F, big, nullptr) == K3MOE_EINVAL);
  CHECK(k3moe_router(&K3, 1, nullptr, 0, Fu16, nullptr, ids, gates, F, big, nullptr) ==
        K3MOE_EINVAL);
  CHECK(k3moe_router(&K3, 1, F_odd, 0, Fu16, nullptr, ids, gates, F, big, nullptr) ==
        K3MOE_EINVAL);
  CHECK(k3moe_router(&K3, 1, F, 0, nullptr, nullptr, ids, gates, F, big, nullptr) ==
        K3MOE_EINVAL);
  CHECK(k3moe_router(&K3, 1, F, 0, Fu16, nullptr, nullptr, gates, F, big, nullptr) ==
        K3MOE_EINVAL);
  CHECK(k3moe_router(&K3, 1, F, 0, Fu16, nullptr, ids, gates, F, 64, nullptr) ==
        K3MOE_EWORKSPACE && has_msg());
  CHECK(k3moe_router(&K3, 1, F, 0, Fu16, nullptr, ids, gates, nullptr, big, nullptr) ==
        K3MOE_EINVAL);
  // bucket
  CHECK(k3moe_route_bucket(&K3, 5, nullptr, ids, ids, F, big, nullptr) == K3MOE_EINVAL);
  CHECK(k3moe_route_bucket(&K3, 5, ids, ids, ids, F, 16, nullptr) == K3MOE_EWORKSPACE);
  CHECK(k3moe_route_bucket(&K3, 0, nullptr, nullptr, nullptr, nullptr, 0, nullptr) == K3MOE_OK);
  // experts
  CHECK(k3moe_expert_ffn(&K3, 3, F, 0, nullptr, ids, ids, gates, y, F, big, nullptr) ==
        K3MOE_EINVAL);
  {
    k3moe_mx_experts e2 = ex;
    e2.down_q = static_cast<const uint8_t*>(F_odd);
    CHECK(k3moe_expert_ffn(&K3, 3, F, 0, &e2, ids, ids, gates, y, F, big, nullptr) ==
          K3MOE_EINVAL);
    e2 = ex;
    e2.up_s = nullptr;
    CHECK(k3moe_expert_ffn(&K3, 3, F, 0, &e2, ids, ids, gates, y, F, big, nullptr) ==
          K3MOE_EINVAL);
  }
  CHECK(k3moe_expert_ffn(&K3, 3, F, 0, &ex, ids, ids, gates, static_cast<float*>(F_odd), F, big,
                         nullptr) == K3MOE_EINVAL);
  {
    k3moe_dims wide{7168, 32 * 5 * 3, 896, 16};  // d_ff/32 = 15: 15 blocks on one lane
    CHECK(k3moe_expert_ffn(&wide, 3, F, 0, &ex, ids, ids, gates, y, F, big, nullptr) ==
          K3MOE_EUNSUPPORTED && has_msg());
  }
  CHECK(k3moe_expert_ffn(&K3, 3, F, 0, &ex, ids, ids, gates, y, F, 100, nullptr) ==
        K3MOE_EWORKSPACE);
  // layer
  k3moe_block blk{Fu16, 1e-6f, Fu16, Fu16, Fu16};
  CHECK(k3moe_layer_forward(&K3, 1, F, K3MOE_BF16, Fu16, nullptr, &ex, &blk, y, nullptr, nullptr,
                            nullptr, F, big, nullptr) == K3MOE_EINVAL);  // block needs fp32
  blk.rms_eps = -1.0f;
  CHECK(k3moe_layer_forward(&K3, 1, F, K3MOE_F32, Fu16, nullptr, &ex, &blk, y, nullptr, nullptr,
                            nullptr, F, big, nullptr) == K3MOE_EINVAL);
  blk.rms_eps = 1e-6f;
  blk.sh_up = reinterpret_cast<const uint16_t*>(F_odd);
  CHECK(k3moe_layer_forward(&K3, 1, F, K3MOE_F32, Fu16, nullptr, &ex, &blk, y, nullptr, nullptr,
                            nullptr, F, big, nullptr) == K3MOE_EINVAL);
  CHECK(k3moe_layer_forward(&K3, 2048, F, K3MOE_BF16, Fu16, nullptr, &ex, nullptr, y, nullptr,
                            nullptr, nullptr, F, k3moe_workspace_bytes(&K3, 2047), nullptr) ==
        K3MOE_EWORKSPACE);
  // T = 0 is a no-op once dims, T and dtype are valid (no pointer is looked at)
  CHECK(k3moe_layer_forward(&K3, 0, nullptr, 0, nullptr, nullptr, nullptr, nullptr, nullptr,
                            nullptr, nullptr, nullptr, nullptr, 0, nullptr) == K3MOE_OK);

  // slot cache: host-only plan on random streams
  {
    const int E = 64, C = 12, M = 32;
    const size_t n = k3moe_cache_state_bytes(E, C, M);
    CHECK(n > 0);
    std::vector<uint64_t> st(n / 8 + 1);
    CHECK(k3moe_cache_init(st.data(), n - 1, E, C, M) == K3MOE_EWORKSPACE);
    CHECK(k3moe_cache_init(reinterpret_cast<char*>(st.data()) + 4, n, E, C, M) == K3MOE_EINVAL);
    CHECK(k3moe_cache_init(st.data(), n, E, C, M) == K3MOE_OK);
    uint32_t r = 7u;
    std::vector<int32_t> idv(M), slot(M), fetch(2 * C);
    for (int call = 0; call < 500; ++call) {
      const int nid = 1 + int(r % M);
      for (int i = 0; i < nid; ++i) {
        r = r * 1664525u + 1013904223u;
        idv[i] = int((r >> 8) % 12u) + (call % 5) * 6;  // at most 12 distinct per call
      }
      int32_t nf = -1;
      CHECK(k3moe_cache_plan(st.data(), nid, idv.data(), slot.data(), fetch.data(), &nf) ==
            K3MOE_OK);
      CHECK(nf >= 0 && nf <= C);
      for (int i = 0; i < nid; ++i) CHECK(slot[i] >= 0 && slot[i] < C);
      for (int i = 0; i < nid; ++i)
        for (int j = 0; j < nid; ++j) CHECK((idv[i] == idv[j]) == (slot[i] == slot[j]));
    }
    idv[0] = E;
    int32_t nf = 0;
    CHECK(k3moe_cache_plan(st.data(), 1, idv.data(), slot.data(), fetch.data(), &nf) ==
          K3MOE_EINVAL);
    for (int i = 0; i < 13; ++i) idv[i] = i;
    CHECK(k3moe_cache_plan(st.data(), 13, idv.data(), slot.data(), fetch.data(), &nf) ==
          K3MOE_EUNSUPPORTED);
    k3moe_cache_stats cs{};
    CHECK(k3moe_cache_stats_get(st.data(), &cs) == K3MOE_OK && cs.hits + cs.misses > 0);
    CHECK(k3moe_cache_stats_get(st.data(), nullptr) == K3MOE_EINVAL);
  }
  CHECK(k3moe_release() == K3MOE_OK);
  if (fails) {
    std::fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
