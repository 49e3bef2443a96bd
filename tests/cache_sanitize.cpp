// Host-only driver of the expert slot cache (expert_cache.cpp), built by
// tests/test_cache_sanitize.py with AddressSanitizer and UndefinedBehaviorSanitizer:
// random routing streams over several cache shapes, checking after every call that each
// routed expert sits in the slot returned for it and that no slot holds two experts.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "k3moe_cache.h"

static uint32_t rng_state = 12345u;
static uint32_t rnd() {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 17;
  rng_state ^= rng_state << 5;
  return rng_state;
}

int main() {
  const int shapes[][3] = {{1, 1, 1}, {8, 3, 5}, {40, 12, 12}, {896, 64, 64}, {33, 33, 40}};
  long calls = 0, errors = 0;
  for (const auto& sh : shapes) {
    const int E = sh[0], C = sh[1], max_ids = sh[2];
    const size_t n = k3moe::cache_state_bytes(E, C, max_ids);
    if (n == 0) return 2;
    std::vector<uint64_t> buf(n / 8 + 1);
    if (k3moe::cache_init(buf.data(), n, E, C, max_ids) != 0) return 3;
    if (k3moe::cache_init(buf.data(), n - 1, E, C, max_ids) != -3) return 4;
    if (k3moe::cache_init(buf.data(), n, E, C, max_ids) != 0) return 5;
    k3moe::CacheView v = k3moe::cache_view(buf.data());
    std::vector<int32_t> ids(max_ids), slots(max_ids), fetch(2 * C);
    std::vector<int32_t> owner(C);
    for (int it = 0; it < 4000; ++it) {
      const int m = 1 + (int)(rnd() % (uint32_t)max_ids);
      for (int i = 0; i < m; ++i) {
        // mostly valid ids, a few out of range to exercise the error path
        ids[i] = (rnd() % 97u == 0u) ? (int32_t)(E + (rnd() % 3u)) : (int32_t)(rnd() % (uint32_t)E);
      }
      int32_t nf = 0, nd = 0;
      const int rc = k3moe::cache_plan(v, m, ids.data(), slots.data(), fetch.data(), &nf, &nd);
      ++calls;
      if (rc != 0) {
        ++errors;
        continue;
      }
      for (int s = 0; s < C; ++s) owner[s] = -1;
      for (int i = 0; i < m; ++i) {
        const int s = slots[i];
        if (s < 0 || s >= C) return 10;
        if (owner[s] >= 0 && owner[s] != ids[i]) return 11;  // two experts in one slot
        owner[s] = ids[i];
        if (v.slot_of[ids[i]] != s || v.expert_of[s] != ids[i]) return 12;
      }
      for (int i = 0; i < nf; ++i)
        if (fetch[2 * i] < 0 || fetch[2 * i] >= E || fetch[2 * i + 1] < 0 || fetch[2 * i + 1] >= C)
          return 13;
    }
  }
  std::printf("calls %ld errors %ld ok\n", calls, errors);
  return 0;
}
