// k3moe_cache.h — host-side expert slot cache (internal; expert_cache.cpp).
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace k3moe {

// Head of the caller-owned state buffer; arrays follow (see expert_cache.cpp).
struct CacheHeader {
  uint32_t magic;
  int32_t n_experts, n_slots, max_ids;
  uint64_t clock;                 // one tick per planned call
  int64_t hits, misses, bytes;    // cumulative
};

struct CacheView {
  CacheHeader* h;          // nullptr if the buffer is not an initialised state
  int32_t* slot_of;        // [E] slot of each expert, -1 if not resident
  int32_t* expert_of;      // [C] expert in each slot, -1 if empty
  uint64_t* last_use;      // [C] clock of the last call that used the slot (0 = never)
  uint64_t* mark;          // [E] per-call marks
  int32_t* ids;            // [max_ids] host copy of routed ids
  int32_t* slots;          // [max_ids] their slots
  int32_t* fetch;          // [2 C] (expert, slot) per miss
};

size_t cache_state_bytes(int32_t E, int32_t C, int32_t max_ids);
// 0, or -1 (bad arguments or buffer not 8-byte aligned), -3 (buffer too small).
int cache_init(void* state, size_t bytes, int32_t E, int32_t C, int32_t max_ids);
CacheView cache_view(void* state);
// 0, or -1 (an id outside [0, E)), -2 (more distinct experts than slots; state unchanged
// apart from per-call marks).
int cache_plan(CacheView& v, int32_t n, const int32_t* ids, int32_t* slot_ids, int32_t* fetch,
               int32_t* n_fetch, int32_t* n_distinct);

}  // namespace k3moe
