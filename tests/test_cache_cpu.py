"""Host-side expert slot cache (k3moe_cache_*): the plan checked against a direct model of
its policy on random routing streams, its invariants and its error paths. No GPU."""
import ctypes

import numpy as np
import pytest

import mxfp4_expert_matmul_k3moe_amd as k3


class LRUModel:
    """The documented policy written out: hits keep their slot; each missing expert, in order
    of first appearance, takes the slot this call does not use with the oldest last use
    (lowest slot index among equals; never-used slots count as oldest)."""

    def __init__(self, E, C):
        self.C = C
        self.slot_of = {}
        self.expert_of = [-1] * C
        self.last = [0] * C
        self.t = 0
        self.hits = self.misses = 0

    def plan(self, ids):
        distinct = list(dict.fromkeys(int(e) for e in ids))
        assert len(distinct) <= self.C
        self.t += 1
        for e in distinct:
            if e in self.slot_of:
                self.last[self.slot_of[e]] = self.t
                self.hits += 1
        fetch = []
        for e in distinct:
            if e in self.slot_of:
                continue
            v = min((s for s in range(self.C) if self.last[s] < self.t),
                    key=lambda s: (self.last[s], s))
            old = self.expert_of[v]
            if old >= 0:
                del self.slot_of[old]
            self.expert_of[v] = e
            self.slot_of[e] = v
            self.last[v] = self.t
            fetch.append((e, v))
            self.misses += 1
        return [self.slot_of[int(e)] for e in ids], fetch


@pytest.mark.parametrize("E,C,k,Tmax,seed", [(40, 12, 4, 3, 1), (32, 4, 4, 1, 2),
                                              (896, 64, 16, 4, 3), (8, 8, 2, 6, 4)])
def test_plan_matches_policy_model(E, C, k, Tmax, seed):
    rng = np.random.default_rng(seed)
    cache = k3.ExpertCache(E, C, Tmax * k)
    model = LRUModel(E, C)
    hot = rng.permutation(E)[: max(C // 2, 1)]  # some locality, so hits happen
    for _ in range(300):
        T = int(rng.integers(1, Tmax + 1))
        rows = []
        for _t in range(T):
            pool = hot if rng.random() < 0.5 and len(hot) >= k else np.arange(E)
            rows.append(rng.choice(pool, size=k, replace=False))
        ids = np.concatenate(rows).astype(np.int32)
        if len(set(ids.tolist())) > C:
            with pytest.raises(k3.K3MoEError) as ei:
                cache.plan(ids)
            assert ei.value.code == k3.EUNSUPPORTED
            continue
        slots, fetch = cache.plan(ids)
        ms, mf = model.plan(ids)
        assert slots.tolist() == ms and fetch == mf
        # every routed expert now sits in the slot it was given, one expert per slot
        assert len(set(zip(ids.tolist(), slots.tolist()))) == len(set(ids.tolist()))
    st = cache.stats()
    assert (st.hits, st.misses) == (model.hits, model.misses)
    assert st.hits > 0 and st.misses > 0


def test_plan_errors_and_state_checks():
    cache = k3.ExpertCache(10, 3, 8)
    with pytest.raises(k3.K3MoEError) as ei:
        cache.plan([1, 10])  # id out of range
    assert ei.value.code == k3.EINVAL
    with pytest.raises(k3.K3MoEError) as ei:
        cache.plan([0, 1, 2, 3])  # four distinct experts, three slots
    assert ei.value.code == k3.EUNSUPPORTED
    slots, fetch = cache.plan([4, 4, 5])  # repeated ids share one slot
    assert slots[0] == slots[1] != slots[2] and len(fetch) == 2
    L = k3.lib()
    assert L.k3moe_cache_state_bytes(10, 11, 8) == 0  # more slots than experts
    assert L.k3moe_cache_state_bytes(10, 0, 8) == 0
    n = L.k3moe_cache_state_bytes(10, 3, 8)
    buf = np.zeros(n // 8 + 2, dtype=np.uint64)
    p = buf.ctypes.data
    assert L.k3moe_cache_init(ctypes.c_void_p(p), n - 1, 10, 3, 8) == k3.EWORKSPACE
    assert L.k3moe_cache_init(ctypes.c_void_p(p + 4), n, 10, 3, 8) == k3.EINVAL  # misaligned
    assert L.k3moe_cache_init(ctypes.c_void_p(p), n, 10, 3, 8) == k3.OK
    junk = np.zeros(64, dtype=np.uint64)
    nf = ctypes.c_int32(0)
    ids = np.zeros(1, dtype=np.int32)
    assert L.k3moe_cache_plan(ctypes.c_void_p(junk.ctypes.data), 1,
                              ctypes.c_void_p(ids.ctypes.data), ctypes.c_void_p(ids.ctypes.data),
                              ctypes.c_void_p(ids.ctypes.data), ctypes.byref(nf)) == k3.EINVAL
