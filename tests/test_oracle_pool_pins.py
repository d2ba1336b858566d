"""Pins of the oracle's residency-policy simulator against textbook caches,
exhaustive optimal (Belady) search on tiny traces, and the cache hit-rate
ceiling of the local-inference explainer (step 4: no policy beats the sum of
the probabilities of the experts that fit)."""
import itertools
from collections import OrderedDict

import numpy as np
import pytest

import oracle as O


def _trace(rng, n, E, k, L=1, p=None):
    layers = rng.integers(0, L, n).astype(np.int32)
    ids = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(n)]).astype(np.int32)
    return layers, ids


def _textbook_lru(E, C, k, ids):
    """OrderedDict LRU.  Within one event the hits are touched first (ascending
    id), then the misses are inserted (ascending id); this way a miss never
    evicts an expert the same event needs."""
    cache = OrderedDict((e, None) for e in range(C))
    misses, evicts = [], []
    for R in ids:
        R = sorted(int(e) for e in R)
        hit = [e for e in R if e in cache]
        mis = [e for e in R if e not in cache]
        for e in hit:
            cache.move_to_end(e)
        ev = []
        for e in mis:
            victim = next(iter(cache))
            del cache[victim]
            cache[e] = None
            ev.append(victim)
        misses.append(mis)
        evicts.append(ev)
    return misses, evicts


def _textbook_lfu(E, C, k, ids):
    """LFU with LRU tie-break; frequencies count every routed access, also of
    non-resident experts (the counter lives per expert, not per slot)."""
    freq = np.zeros(E, np.int64)
    last = {e: e - C for e in range(C)}
    cache = set(range(C))
    clock = 0
    misses, evicts = [], []
    for R in ids:
        R = sorted(int(e) for e in R)
        for e in R:
            freq[e] += 1
        mis = []
        ev = []
        for e in R:
            if e in cache:
                clock += 1
                last[e] = clock
        for e in R:
            if e in cache:
                continue
            cand = [c for c in cache if c not in R]
            victim = min(cand, key=lambda c: (freq[c], last[c], c))
            cache.remove(victim)
            cache.add(e)
            clock += 1
            last[e] = clock
            mis.append(e)
            ev.append(victim)
        misses.append(mis)
        evicts.append(ev)
    return misses, evicts


def _lists(ml, el):
    return ([[int(e) for e in row if e >= 0] for row in ml],
            [[int(e) for e in row if e >= 0] for row in el])


@pytest.mark.parametrize("seed", range(4))
def test_shift0_is_textbook_lru(seed):
    rng = np.random.default_rng(seed)
    E, C, k = 16, 6, 3
    layers, ids = _trace(rng, 400, E, k)
    h, m, ml, el = O.pool_sim(1, E, C, 0, k, layers, ids)
    tm, te = _textbook_lru(E, C, k, ids)
    assert _lists(ml, el) == (tm, te)
    assert np.array_equal(h + m, np.full(len(ids), k))


@pytest.mark.parametrize("seed", range(4))
def test_no_decay_is_textbook_lfu(seed):
    rng = np.random.default_rng(100 + seed)
    E, C, k = 12, 5, 2
    p = np.arange(1, E + 1, dtype=np.float64) ** -1.0
    p /= p.sum()
    layers, ids = _trace(rng, 300, E, k, p=p)
    h, m, ml, el = O.pool_sim(1, E, C, -1, k, layers, ids)
    tm, te = _textbook_lfu(E, C, k, ids)
    assert _lists(ml, el) == (tm, te)


def test_full_capacity_never_misses():
    rng = np.random.default_rng(0)
    E, k, L = 64, 8, 4
    layers, ids = _trace(rng, 500, E, k, L)
    h, m, _, _ = O.pool_sim(L, E, E, 3, k, layers, ids)
    assert m.sum() == 0 and h.sum() == 500 * k


def test_layers_are_independent():
    rng = np.random.default_rng(9)
    E, C, k = 10, 4, 2
    la, ia = _trace(rng, 50, E, k)
    lb, ib = _trace(rng, 50, E, k)
    _, ma, mla, ela = O.pool_sim(1, E, C, 3, k, la, ia)
    _, mb, mlb, elb = O.pool_sim(1, E, C, 3, k, lb, ib)
    # interleave the two traces on two layers, each keeping its own order
    layers = rng.permutation(np.repeat(np.array([0, 1], np.int32), 50))
    ids = np.empty((100, k), np.int32)
    ids[layers == 0] = ia
    ids[layers == 1] = ib
    _, m2, ml2, el2 = O.pool_sim(2, E, C, 3, k, layers, ids)
    assert np.array_equal(m2[layers == 0], ma) and np.array_equal(m2[layers == 1], mb)
    assert np.array_equal(el2[layers == 0], ela) and np.array_equal(el2[layers == 1], elb)


def _belady_min(E, C, k, ids):
    """Exhaustive optimum: the fewest misses any policy can reach when it keeps
    C experts, must hold the whole routed set at each event, starts from
    experts 0..C-1 and evicts only non-routed residents."""
    best = [10 ** 9]
    memo = {}

    def go(i, cache):
        if i == len(ids):
            return 0
        key = (i, cache)
        if key in memo:
            return memo[key]
        R = set(int(e) for e in ids[i])
        mis = [e for e in R if e not in cache]
        cand = [c for c in cache if c not in R]
        res = 10 ** 9
        for victims in itertools.combinations(sorted(cand), len(mis)):
            nc = frozenset((cache - set(victims)) | set(mis))
            res = min(res, len(mis) + go(i + 1, nc))
        memo[key] = res
        return res

    return go(0, frozenset(range(C)))


@pytest.mark.parametrize("seed", range(6))
def test_misses_at_least_belady_and_compulsory(seed):
    rng = np.random.default_rng(200 + seed)
    E, C, k = 6, 3, 2
    layers, ids = _trace(rng, 12, E, k)
    opt = _belady_min(E, C, k, ids)
    touched = set(int(e) for e in ids.reshape(-1))
    compulsory = len(touched - set(range(C)))
    for shift in (-1, 0, 1, 3):
        _, m, _, _ = O.pool_sim(1, E, C, shift, k, layers, ids)
        assert m.sum() >= opt >= compulsory


def test_hit_rate_below_ceiling_iid():
    """iid Zipf traces: no online policy exceeds the expected hit ceiling of
    keeping the C experts most likely to be routed (sum of their inclusion
    probabilities / k)."""
    rng = np.random.default_rng(42)
    E, C, k, n = 64, 30, 8, 6000
    p = np.arange(1, E + 1, dtype=np.float64) ** -1.0
    p /= p.sum()
    layers, ids = _trace(rng, n, E, k, p=p)
    incl = np.bincount(ids.reshape(-1), minlength=E) / n       # empirical inclusion
    ceiling = np.sort(incl)[::-1][:C].sum() / k
    for shift in (0, 3, -1):
        h, m, _, _ = O.pool_sim(1, E, C, shift, k, layers, ids)
        assert h.sum() / (n * k) <= ceiling + 1e-12
    # uniform routing: every policy collapses to about C/E
    layers, ids = _trace(rng, n, E, k)
    h, m, _, _ = O.pool_sim(1, E, C, 3, k, layers, ids)
    assert abs(h.sum() / (n * k) - C / E) < 0.03


def test_rejects_bad_capacity():
    with pytest.raises(ValueError):
        O.pool_sim(1, 8, 1, 3, 2, np.zeros(1, np.int32), np.array([[0, 1]], np.int32))
    with pytest.raises(ValueError):
        O.pool_sim(1, 8, 9, 3, 2, np.zeros(1, np.int32), np.array([[0, 1]], np.int32))


# --------------------------------------------- profile-pinned policy

def test_profile_pin_brute_force_with_ties():
    rng = np.random.default_rng(3)
    for _ in range(50):
        L, E, C = 3, 10, 4
        counts = rng.integers(0, 4, (L, E))          # many ties
        got = O.profile_pin(counts, C)
        for l in range(L):
            want = sorted(sorted(range(E), key=lambda e: (-counts[l, e], e))[:C])
            assert list(got[l]) == want


def test_pinned_sim_is_set_membership():
    rng = np.random.default_rng(4)
    L, E, k, C = 2, 12, 3, 5
    pinned = np.stack([np.sort(rng.choice(E, C, replace=False)) for _ in range(L)])
    layers, ids = _trace(rng, 200, E, k, L=L)
    h, m, ml = O.pool_sim_pinned(L, E, pinned, k, layers, ids)
    for i, (l, R) in enumerate(zip(layers, ids)):
        P = set(int(e) for e in pinned[l])
        mis = sorted(set(int(e) for e in R) - P)
        assert h[i] == len(set(int(e) for e in R) & P) and m[i] == len(mis)
        assert list(ml[i][:len(mis)]) == mis and all(ml[i][len(mis):] == -1)
    # every expert pinned: no misses at all
    full = np.tile(np.arange(E, dtype=np.int32), (L, 1))
    h, m, _ = O.pool_sim_pinned(L, E, full, k, layers, ids)
    assert m.sum() == 0 and h.sum() == ids.size


def test_pinned_by_own_profile_equals_static_ceiling():
    """Pinning the C most counted experts of the very trace it replays gives
    exactly the summed counts of those experts: the ceiling of any fixed set."""
    rng = np.random.default_rng(5)
    E, C, k, n = 64, 30, 8, 3000
    p = np.arange(1, E + 1, dtype=np.float64) ** -1.0
    p /= p.sum()
    layers, ids = _trace(rng, n, E, k, p=p)
    counts = np.bincount(ids.reshape(-1), minlength=E)[None, :]
    h, m, _ = O.pool_sim_pinned(1, E, O.profile_pin(counts, C), k, layers, ids)
    assert h.sum() == np.sort(counts[0])[::-1][:C].sum()


def _zipf_trace(rng, n, E, k, perm):
    p = np.arange(1, E + 1, dtype=np.float64) ** -1.0
    p /= p.sum()
    q = np.empty(E)
    q[perm] = p                                   # expert perm[r] has rank r + 1
    return _trace(rng, n, E, k, p=q)


def test_profile_wins_stable_load_lru_wins_shifted_load():
    """The explainer's comparison: with a stable workload a measured profile
    beats recency (and sits at the ceiling); when the workload changes after
    the profile was taken, the profile is stale and recency wins."""
    rng = np.random.default_rng(6)
    E, C, k = 64, 30, 8
    pa, pb = rng.permutation(E), rng.permutation(E)
    _, prof_ids = _zipf_trace(rng, 3000, E, k, pa)
    counts = np.bincount(prof_ids.reshape(-1), minlength=E)[None, :]
    pinned = O.profile_pin(counts, C)
    # stable: same distribution as the profile
    layers, ids = _zipf_trace(rng, 4000, E, k, pa)
    hp, _, _ = O.pool_sim_pinned(1, E, pinned, k, layers, ids)
    hl, _, _, _ = O.pool_sim(1, E, C, 0, k, layers, ids)
    incl = np.bincount(ids.reshape(-1), minlength=E) / len(ids)
    ceiling = np.sort(incl)[::-1][:C].sum() / k
    rate_p, rate_l = hp.sum() / ids.size, hl.sum() / ids.size
    assert rate_p > rate_l
    assert ceiling - 0.01 <= rate_p <= ceiling + 1e-12
    # shifted: the hot set moves after the profile
    layers, ids = _zipf_trace(rng, 4000, E, k, pb)
    hp, _, _ = O.pool_sim_pinned(1, E, pinned, k, layers, ids)
    hl, _, _, _ = O.pool_sim(1, E, C, 0, k, layers, ids)
    assert hl.sum() > hp.sum()
