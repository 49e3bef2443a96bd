// expert_cache.cpp — residency of routed experts beyond HBM: the host-side slot cache.
//
// The routed experts are never kept whole in fast memory: the ones a token selects are read
// on demand from slower storage and multiplied in their packed form ("用纯C语言把1.56TB的
// Kimi K3模型塞进8GB内存运行", kongchang.com, section 专家权重永不常驻内存; project card
// "P053 FareedKhan-dev/kimi-k3-in-c", core features: expert streaming), and recently used
// expert weights are kept in an LRU cache ("Kimi K3 纯 C 语言 CPU 推理实战",
// chenxutan.com/d/5901.html, §3.3 分块加载与缓存复用). Here all E experts of a layer stay in
// pinned host memory and n_slots expert slots live in HBM; this file holds the bookkeeping
// that maps experts to slots. Policy: an expert already in a slot keeps it (hit); a missing
// expert takes the least recently used slot that the current call does not use, lowest
// slot index first among equals (miss). Pure host code: no GPU calls.
#include "k3moe_cache.h"

#include <cstring>

namespace k3moe {
namespace {

constexpr uint32_t kMagic = 0x434D334Bu;  // "K3MC"

size_t align8(size_t v) { return (v + 7) / 8 * 8; }

struct Offsets {
  size_t slot_of, expert_of, last_use, mark, ids, slots, fetch, total;
};

Offsets offsets_for(int32_t E, int32_t C, int32_t max_ids) {
  Offsets o;
  size_t p = align8(sizeof(CacheHeader));
  o.slot_of = p;   p = align8(p + (size_t)E * 4);
  o.expert_of = p; p = align8(p + (size_t)C * 4);
  o.last_use = p;  p = align8(p + (size_t)C * 8);
  o.mark = p;      p = align8(p + (size_t)E * 8);
  o.ids = p;       p = align8(p + (size_t)max_ids * 4);
  o.slots = p;     p = align8(p + (size_t)max_ids * 4);
  o.fetch = p;     p = align8(p + (size_t)C * 8);
  o.total = p;
  return o;
}

}  // namespace

size_t cache_state_bytes(int32_t E, int32_t C, int32_t max_ids) {
  if (E < 1 || C < 1 || C > E || max_ids < 1) return 0;
  return offsets_for(E, C, max_ids).total;
}

int cache_init(void* state, size_t bytes, int32_t E, int32_t C, int32_t max_ids) {
  const size_t need = cache_state_bytes(E, C, max_ids);
  if (need == 0 || !state || (reinterpret_cast<uintptr_t>(state) & 7u)) return -1;
  if (bytes < need) return -3;
  std::memset(state, 0, need);
  CacheHeader* h = static_cast<CacheHeader*>(state);
  h->magic = kMagic;
  h->n_experts = E;
  h->n_slots = C;
  h->max_ids = max_ids;
  CacheView v = cache_view(state);
  for (int32_t e = 0; e < E; ++e) v.slot_of[e] = -1;
  for (int32_t s = 0; s < C; ++s) v.expert_of[s] = -1;
  return 0;
}

CacheView cache_view(void* state) {
  CacheView v{};
  CacheHeader* h = static_cast<CacheHeader*>(state);
  if (!h || h->magic != kMagic) return v;
  const Offsets o = offsets_for(h->n_experts, h->n_slots, h->max_ids);
  char* b = static_cast<char*>(state);
  v.h = h;
  v.slot_of = reinterpret_cast<int32_t*>(b + o.slot_of);
  v.expert_of = reinterpret_cast<int32_t*>(b + o.expert_of);
  v.last_use = reinterpret_cast<uint64_t*>(b + o.last_use);
  v.mark = reinterpret_cast<uint64_t*>(b + o.mark);
  v.ids = reinterpret_cast<int32_t*>(b + o.ids);
  v.slots = reinterpret_cast<int32_t*>(b + o.slots);
  v.fetch = reinterpret_cast<int32_t*>(b + o.fetch);
  return v;
}

int cache_plan(CacheView& v, int32_t n, const int32_t* ids, int32_t* slot_ids, int32_t* fetch,
               int32_t* n_fetch, int32_t* n_distinct) {
  CacheHeader& h = *v.h;
  const int32_t E = h.n_experts, C = h.n_slots;
  // epoch t: slots with last_use == t are used by this call; mark 2t = counted, 2t+1 = placed
  const uint64_t t = ++h.clock;
  const uint64_t seen = 2 * t, placed = 2 * t + 1;
  int32_t distinct = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t e = ids[i];
    if (e < 0 || e >= E) return -1;
    if (v.mark[e] != seen) {
      v.mark[e] = seen;
      ++distinct;
    }
  }
  if (distinct > C) return -2;
  int32_t nf = 0, hits = 0;
  for (int32_t i = 0; i < n; ++i) {  // hits first: they keep their slots
    const int32_t e = ids[i];
    if (v.mark[e] == seen && v.slot_of[e] >= 0) {
      v.mark[e] = placed;
      v.last_use[v.slot_of[e]] = t;
      ++hits;
    }
  }
  for (int32_t i = 0; i < n; ++i) {  // misses in order of first appearance
    const int32_t e = ids[i];
    if (v.mark[e] != seen) continue;
    v.mark[e] = placed;
    int32_t vic = -1;
    uint64_t best = ~0ull;
    for (int32_t s = 0; s < C; ++s)
      if (v.last_use[s] < t && v.last_use[s] < best) {
        best = v.last_use[s];
        vic = s;
      }
    // distinct <= C guarantees a slot this call does not use
    const int32_t old = v.expert_of[vic];
    if (old >= 0) v.slot_of[old] = -1;
    v.expert_of[vic] = e;
    v.slot_of[e] = vic;
    v.last_use[vic] = t;
    fetch[2 * nf] = e;
    fetch[2 * nf + 1] = vic;
    ++nf;
  }
  for (int32_t i = 0; i < n; ++i) slot_ids[i] = v.slot_of[ids[i]];
  h.hits += hits;
  h.misses += nf;
  *n_fetch = nf;
  if (n_distinct) *n_distinct = distinct;
  return 0;
}

}  // namespace k3moe
