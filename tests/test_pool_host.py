"""The slot pool's contract on the CPU, through the host-only build of the
same pool code (libmoe_pool_host.so: host memory slots, memcpy copies,
injectable copy failures).  Policy decisions are checked against the
oracle's independent simulator; the generation protocol against the
resident-qpacked-cache-v1 rules (Horizon RunMap "03 / Arquitetura"):
the source is never written, a miss lands in a spare slot, the previous
generation stays intact until the new one is published, a failure before
publication keeps the previous generation, capacity is fixed up front."""
import ctypes as C
import os

import numpy as np
import pytest

import int4_weight_only_router_amd as M
from int4_weight_only_router_amd import build as B
import oracle as O


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.POOL_HOST_LIB) or not B.up_to_date():
        B.build()
    lib = C.CDLL(B.POOL_HOST_LIB)
    vp = C.c_void_p
    lib.moe_pool_create.argtypes = [C.POINTER(M.PoolConfig), vp, C.POINTER(vp)]
    lib.moe_pool_prepare.argtypes = [vp, C.c_int, vp, C.c_int, vp, C.POINTER(vp),
                                     C.POINTER(M.PoolStats)]
    lib.moe_pool_retire.argtypes = [vp, C.c_int, vp]
    lib.moe_pool_stats.argtypes = [vp, C.POINTER(M.PoolStats)]
    lib.moe_pool_access_counts.argtypes = [vp, vp, vp]
    lib.moe_pool_reset.argtypes = [vp]
    lib.moe_pool_destroy.argtypes = [vp]
    lib.moe_pool_fake_fail_after.argtypes = [vp, C.c_long]
    lib.moe_pool_pin.argtypes = [vp, C.c_int, vp, C.c_int]
    lib.moe_pool_fake_set_delay.argtypes = [vp, C.c_int]
    lib.moe_pool_fake_complete_copies.argtypes = [vp]
    lib.moe_pool_fake_complete_copies.restype = C.c_long
    lib.moe_pool_fake_pending.argtypes = [vp]
    lib.moe_pool_fake_pending.restype = C.c_long
    lib.moe_pool_fake_pending_dst.argtypes = [vp, C.c_long]
    lib.moe_pool_fake_pending_dst.restype = C.c_void_p
    lib.moe_last_error.restype = C.c_char_p
    return lib


class FakePool:
    def __init__(self, lib, Lyr, E, k, Cap, S, shift, nbytes=512, seed=0):
        self.lib, self.L, self.E, self.k, self.nbytes = lib, Lyr, E, k, nbytes
        rng = np.random.default_rng(seed)
        self.src = rng.integers(0, 256, (Lyr, E, nbytes), dtype=np.uint8)
        self.src_copy = self.src.copy()
        ptrs = (C.c_void_p * (Lyr * E))(*[self.src[l, e].ctypes.data
                                          for l in range(Lyr) for e in range(E)])
        cfg = M.PoolConfig(layers=Lyr, experts=E, topk=k, capacity=Cap, spares=S,
                           decay_shift=shift, expert_bytes=nbytes)
        self.h = C.c_void_p()
        self.rc = lib.moe_pool_create(C.byref(cfg), C.cast(ptrs, C.c_void_p), C.byref(self.h))

    def prepare(self, layer, ids):
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        tab = C.c_void_p()
        st = M.PoolStats()
        rc = self.lib.moe_pool_prepare(self.h, layer, ids.ctypes.data, ids.size, None,
                                       C.byref(tab), C.byref(st))
        return rc, tab.value, st

    def retire(self, layer):
        return self.lib.moe_pool_retire(self.h, layer, None)

    def table(self, addr):
        return list((C.c_void_p * self.E).from_address(addr))

    def slot_bytes(self, ptr):
        return np.frombuffer((C.c_uint8 * self.nbytes).from_address(ptr), dtype=np.uint8)

    def stats(self):
        st = M.PoolStats()
        assert self.lib.moe_pool_stats(self.h, C.byref(st)) == 0
        return st

    def access(self):
        h = np.full((self.L, self.E), -1, np.int64)
        m = np.full((self.L, self.E), -1, np.int64)
        assert self.lib.moe_pool_access_counts(self.h, h.ctypes.data, m.ctypes.data) == 0
        return h, m

    def close(self):
        self.lib.moe_pool_destroy(self.h)


def _trace(seed, n, Lyr, E, k, s=1.0):
    rng = np.random.default_rng(seed)
    p = np.arange(1, E + 1, dtype=np.float64) ** -s
    p /= p.sum()
    layers = rng.integers(0, Lyr, n).astype(np.int32)
    ids = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(n)]).astype(np.int32)
    return layers, ids


@pytest.mark.parametrize("shift", [3, 0, -1])
def test_pool_matches_simulator_and_tables_are_complete(L, shift):
    Lyr, E, k, Cap, S = 2, 16, 3, 6, 3
    P = FakePool(L, Lyr, E, k, Cap, S, shift)
    assert P.rc == 0
    layers, ids = _trace(7, 300, Lyr, E, k)
    hits, misses, ml, el = O.pool_sim(Lyr, E, Cap, shift, k, layers, ids)
    prev = {}
    for i, (l, R) in enumerate(zip(layers, ids)):
        rc, tab, st = P.prepare(int(l), R)
        assert rc == 0, L.moe_last_error()
        assert (st.hits, st.misses, st.evictions) == (hits[i], misses[i], misses[i])
        assert st.h2d_bytes == misses[i] * P.nbytes
        t = P.table(tab)
        # a complete generation: exactly C resident experts, every routed one
        assert sum(p is not None for p in t) == Cap
        for e in R:
            assert t[e] is not None
        for e, ptr in enumerate(t):
            if ptr is not None:
                assert np.array_equal(P.slot_bytes(ptr), P.src[l, e])
        # the previous generation's table is untouched by this prepare; a
        # generation with misses gets a table of its own, an all-hit one
        # republishes the current table (same experts, same slots)
        if int(l) in prev:
            old_addr, old_entries = prev[int(l)]
            assert (old_addr != tab) == (misses[i] > 0)
            assert P.table(old_addr) == old_entries
        # evicted experts are gone from the new table
        for v in el[i]:
            if v >= 0:
                assert t[v] is None
        prev[int(l)] = (tab, t)
        assert P.retire(int(l)) == 0
    tot = P.stats()
    assert (tot.hits, tot.misses) == (hits.sum(), misses.sum())
    assert tot.h2d_bytes == misses.sum() * P.nbytes
    assert tot.generation == len(ids)
    assert np.array_equal(P.src, P.src_copy)   # the source is never written
    # per-(layer, expert) access counts: every routed expert of an event is a
    # use; the simulator's miss list of the event names the misses
    uses = np.zeros((Lyr, E), np.int64)
    miss = np.zeros((Lyr, E), np.int64)
    for l, R, m in zip(layers, ids, ml):
        uses[l, R] += 1
        for e in m:
            if e >= 0:
                miss[l, e] += 1
    ah, am = P.access()
    assert np.array_equal(am, miss)
    assert np.array_equal(ah, uses - miss)
    assert L.moe_pool_reset(P.h) == 0
    ah, am = P.access()
    assert not ah.any() and not am.any()
    assert L.moe_pool_access_counts(P.h, None, am.ctypes.data) == M.MOE_EINVAL
    P.close()


def test_full_capacity_has_no_misses(L):
    P = FakePool(L, 1, 8, 2, 8, 2, 3)
    layers, ids = _trace(1, 50, 1, 8, 2)
    for l, R in zip(layers, ids):
        rc, tab, st = P.prepare(int(l), R)
        assert rc == 0 and st.misses == 0
        P.retire(int(l))
    assert P.stats().h2d_bytes == 0
    P.close()


def test_order_errors(L):
    P = FakePool(L, 1, 8, 2, 4, 2, 3)
    assert P.retire(0) == M.MOE_ESTATE
    rc, _, _ = P.prepare(0, [0, 5])
    assert rc == 0
    rc, _, _ = P.prepare(0, [1, 2])
    assert rc == M.MOE_ESTATE
    assert P.retire(0) == 0
    rc, _, _ = P.prepare(0, [9, 1])
    assert rc == M.MOE_EINVAL
    P.close()


def test_capacity_rejections_keep_state(L):
    P = FakePool(L, 1, 12, 2, 4, 2, 3)
    before = P.stats()
    rc, _, _ = P.prepare(0, [4, 5, 6, 7, 8])     # 5 distinct experts > C = 4
    assert rc == M.MOE_ECAPACITY
    rc, _, _ = P.prepare(0, [4, 5, 6])           # 3 misses > 2 spares
    assert rc == M.MOE_ECAPACITY
    after = P.stats()
    assert (before.hits, before.misses, before.generation) == \
        (after.hits, after.misses, after.generation)
    rc, tab, st = P.prepare(0, [4, 5])
    assert rc == 0 and st.misses == 2
    P.close()


def test_profile_rejection(L):
    for Cap, S in [(1, 2), (4, 1), (13, 2)]:
        P = FakePool(L, 1, 12, 2, Cap, S, 3)
        assert P.rc == M.MOE_ECAPACITY
        assert b"rejected" in L.moe_last_error()


def test_copy_failure_keeps_previous_generation(L):
    Lyr, E, k, Cap, S = 1, 10, 2, 4, 2
    ref = FakePool(L, Lyr, E, k, Cap, S, 3, seed=3)
    P = FakePool(L, Lyr, E, k, Cap, S, 3, seed=3)
    layers, ids = _trace(11, 40, Lyr, E, k)
    injected = 0
    for l, R in zip(layers, ids):
        rc_r, tab_r, st_r = ref.prepare(0, R)
        assert rc_r == 0
        ref.retire(0)
        before = P.stats()
        if st_r.misses and injected < 5:
            L.moe_pool_fake_fail_after(P.h, 0)      # the next copy fails
            rc, _, _ = P.prepare(0, R)
            assert rc == M.MOE_EHIP
            after = P.stats()
            assert (before.hits, before.misses, before.generation) == \
                (after.hits, after.misses, after.generation)
            L.moe_pool_fake_fail_after(P.h, -1)
            injected += 1
        rc, tab, st = P.prepare(0, R)
        assert rc == 0
        assert (st.hits, st.misses) == (st_r.hits, st_r.misses)
        t, tr = P.table(tab), ref.table(tab_r)
        assert [p is None for p in t] == [p is None for p in tr]
        P.retire(0)
    assert injected == 5
    P.close()
    ref.close()


def test_reset_restores_initial_placement(L):
    P = FakePool(L, 2, 8, 2, 3, 2, 3)
    layers, ids = _trace(5, 30, 2, 8, 2)
    for l, R in zip(layers, ids):
        assert P.prepare(int(l), R)[0] == 0
        P.retire(int(l))
    assert L.moe_pool_reset(P.h) == 0
    st = P.stats()
    assert (st.hits, st.misses, st.generation) == (0, 0, 0)
    rc, tab, st = P.prepare(0, [0, 1])
    assert rc == 0 and st.hits == 2 and st.misses == 0
    P.close()


def _pin(L, P, layer, experts):
    a = np.ascontiguousarray(experts, dtype=np.int32)
    return L.moe_pool_pin(P.h, layer, a.ctypes.data, a.size)


def test_pinned_pool_matches_simulator(L):
    """moe_pool_pin: the profile's C experts stay resident; every other routed
    expert is copied for one generation and dropped at the next (the oracle's
    pinned simulator decides hits and misses)."""
    Lyr, E, k, Cap, S = 2, 16, 3, 6, 3
    P = FakePool(L, Lyr, E, k, Cap, S, 3)
    assert P.rc == 0
    _, prof = _trace(11, 400, Lyr, E, k)
    prof_layers, _ = _trace(11, 400, Lyr, E, k)
    counts = np.zeros((Lyr, E), np.int64)
    for l, R in zip(prof_layers, prof):
        counts[l, R] += 1
    pinned = O.profile_pin(counts, Cap)
    for l in range(Lyr):
        assert _pin(L, P, l, pinned[l][::-1]) == 0      # any order
    layers, ids = _trace(12, 300, Lyr, E, k)
    hits, misses, ml = O.pool_sim_pinned(Lyr, E, pinned, k, layers, ids)
    for i, (l, R) in enumerate(zip(layers, ids)):
        rc, tab, st = P.prepare(int(l), R)
        assert rc == 0, L.moe_last_error()
        assert (st.hits, st.misses, st.evictions) == (hits[i], misses[i], 0)
        assert st.h2d_bytes == misses[i] * P.nbytes
        t = P.table(tab)
        present = {e for e, ptr in enumerate(t) if ptr is not None}
        assert present == set(int(e) for e in pinned[l]) | set(int(e) for e in R)
        for e in present:
            assert np.array_equal(P.slot_bytes(t[e]), P.src[l, e])
        assert P.retire(int(l)) == 0
    tot = P.stats()
    assert (tot.hits, tot.misses, tot.evictions) == (hits.sum(), misses.sum(), 0)
    assert np.array_equal(P.src, P.src_copy)
    # reset: canonical placement and the decayed-counter policy again
    assert L.moe_pool_reset(P.h) == 0
    h2, m2, _, _ = O.pool_sim(Lyr, E, Cap, 3, k, layers[:50], ids[:50])
    for i in range(50):
        rc, tab, st = P.prepare(int(layers[i]), ids[i])
        assert rc == 0 and (st.hits, st.misses) == (h2[i], m2[i])
        assert P.retire(int(layers[i])) == 0
    P.close()


def test_pin_errors_keep_state(L):
    P = FakePool(L, 1, 8, 2, 4, 2, 3)
    assert _pin(L, P, 0, [0, 1, 2]) == M.MOE_EINVAL          # n != C
    assert _pin(L, P, 0, [0, 1, 2, 2]) == M.MOE_EINVAL       # repeated id
    assert _pin(L, P, 0, [0, 1, 2, 8]) == M.MOE_EINVAL       # out of range
    assert _pin(L, P, 1, [0, 1, 2, 3]) == M.MOE_EINVAL       # no such layer
    rc, _, _ = P.prepare(0, [5, 6])
    assert rc == 0
    assert _pin(L, P, 0, [4, 5, 6, 7]) == M.MOE_ESTATE       # generation not retired
    assert P.retire(0) == 0
    assert _pin(L, P, 0, [4, 5, 6, 7]) == 0
    rc, tab, st = P.prepare(0, [5, 1])
    assert rc == 0 and (st.hits, st.misses) == (1, 1)
    P.close()


@pytest.mark.parametrize("pinned", [False, True])
def test_previous_generation_intact_while_copies_are_in_flight(L, pinned):
    """Copies held back (as if the side stream had not run yet): after each
    prepare, every expert of the previous generation's table still holds its
    source bytes, no queued copy writes into a slot that table references,
    and once the copies land every expert of the new table holds its bytes;
    the victims' slots are reused only after a retire (resident-qpacked-cache-v1:
    readers keep the previous generation until the new one is published).
    Pinned layers: the previous generation's one-off copies (experts outside
    the pinned set) are dropped at the next prepare, after the retire, so
    only the pinned experts' slots are held to this."""
    Lyr, E, k, Cap, S = 2, 12, 3, 5, 3
    P = FakePool(L, Lyr, E, k, Cap, S, 3, nbytes=256, seed=4)
    assert P.rc == 0
    pin_set = set(range(1, 1 + Cap))
    try:
        if pinned:
            for l in range(Lyr):
                assert L.moe_pool_pin(P.h, l, np.arange(1, 1 + Cap, dtype=np.int32).ctypes.data,
                                      Cap) == 0
        assert L.moe_pool_fake_set_delay(P.h, 1) == 0
        layers, ids = _trace(11, 300, Lyr, E, k, s=0.5)
        prev = {}
        for l in range(Lyr):   # the published table of each layer before the trace
            rc, tab, _ = P.prepare(l, np.arange(k, dtype=np.int32) + 1)
            assert rc == 0 and L.moe_pool_fake_complete_copies(P.h) >= 0
            assert P.retire(l) == 0
            prev[l] = P.table(tab)
        in_flight = 0
        for l, R in zip(layers, ids):
            l = int(l)
            rc, tab, st = P.prepare(l, R)
            assert rc == 0, L.moe_last_error()
            npend = L.moe_pool_fake_pending(P.h)
            assert npend == st.misses
            in_flight += npend
            old = [p if (not pinned or e in pin_set) else None for e, p in enumerate(prev[l])]
            old_slots = {p for p in old if p}
            for i in range(npend):
                assert L.moe_pool_fake_pending_dst(P.h, i) not in old_slots
            for e, ptr in enumerate(old):
                if ptr:
                    assert np.array_equal(P.slot_bytes(ptr), P.src[l, e]), (l, e)
            assert L.moe_pool_fake_complete_copies(P.h) == npend
            new = P.table(tab)
            for e in R:
                assert new[int(e)]
            for e, ptr in enumerate(new):
                if ptr:
                    assert np.array_equal(P.slot_bytes(ptr), P.src[l, e]), (l, e)
            assert P.retire(l) == 0
            prev[l] = new
        assert in_flight > 0
        assert np.array_equal(P.src, P.src_copy)
    finally:
        P.close()
