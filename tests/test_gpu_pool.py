"""Expert slot pool (partial residency) on the GPU, through the C ABI.

Horizon RunMap "03 / Arquitetura" (resident-qpacked-cache-v1): the full
INT4 source stays immutable in pinned host memory, misses are copied into
spare HBM slots on a side stream, a complete new generation of the expert
table is published after the copies, and evicted slots are reused only after
their readers retire.  Checks: counters and evictions equal the oracle's
policy simulator on seeded traces; pooled decode reproduces the fully
resident decode bit for bit; the source is never written; H2D bytes equal
misses x blob bytes."""
import numpy as np
import pytest
import torch

import int4_weight_only_router_amd as M
from int4_weight_only_router_amd.layer import MoELayer, blob_table
import moe_inputs as MI
import oracle as O
from tests.gpu_util import DEV, device_experts, f16, say

pytestmark = pytest.mark.gpu


def _pinned_source(cfg, layers):
    """Prepacked blobs of every (layer, expert) copied to pinned host memory."""
    _, total = M.moe_blob_layout(cfg.H, cfg.I, cfg.g)
    src = torch.empty((layers, cfg.E, total), dtype=torch.uint8, pin_memory=True)
    devs = []
    for l in range(layers):
        dev, _ = device_experts(cfg, l)
        src[l].copy_(dev)
        devs.append(dev)
    torch.cuda.synchronize()
    return src, devs, total


def _make_pool(src, cfg, layers, C, S, shift, total):
    ptrs = [src[l, e].data_ptr() for l in range(layers) for e in range(cfg.E)]
    pc = M.PoolConfig(layers=layers, experts=cfg.E, topk=cfg.k, capacity=C, spares=S,
                      decay_shift=shift, expert_bytes=total)
    return M.moe_pool_create(pc, ptrs)


class _DevBuf:
    """A raw device address seen as a uint8 array (read through torch)."""

    def __init__(self, ptr, nbytes):
        self.__cuda_array_interface__ = {"shape": (nbytes,), "typestr": "|u1",
                                         "data": (ptr, False), "version": 3}


def _device_bytes(ptr, nbytes):
    return torch.as_tensor(_DevBuf(ptr, nbytes), device=DEV)


def _zipf_trace(seed, n, L, E, k, s=1.0):
    rng = np.random.default_rng(seed)
    p = np.arange(1, E + 1, dtype=np.float64) ** -s
    p /= p.sum()
    layers = np.tile(np.arange(L, dtype=np.int32), n // L + 1)[:n]
    ids = np.array([rng.choice(E, k, replace=False, p=p) for _ in range(n)], dtype=np.int32)
    return layers, ids


@pytest.mark.parametrize("shift", [3, 0])
def test_pool_counters_match_simulator(shift):
    cfg = MI.TINY
    L, C, S = 3, 4, 2
    say("pool counters tiny shift=%d" % shift)
    src, _, total = _pinned_source(cfg, L)
    before = src.clone()
    pool = _make_pool(src, cfg, L, C, S, shift, total)
    layers, ids = _zipf_trace(1, 240, L, cfg.E, cfg.k)
    hits, misses, ml, el = O.pool_sim(L, cfg.E, C, shift, cfg.k, layers, ids)
    stream = torch.cuda.current_stream()
    try:
        for i, (l, R) in enumerate(zip(layers, ids)):
            tab, st = M.moe_pool_prepare(pool, int(l), np.ascontiguousarray(R), cfg.k, stream)
            assert (st.hits, st.misses, st.evictions) == (hits[i], misses[i], misses[i])
            assert st.h2d_bytes == misses[i] * total
            M.moe_pool_retire(pool, int(l), stream)
            if i % 40 == 0:
                # the published table maps every routed expert to a slot that
                # holds exactly that expert's bytes
                torch.cuda.synchronize()
                t = _device_bytes(tab, cfg.E * 8).view(torch.int64).cpu()
                for e in R:
                    ptr = int(t[int(e)])
                    assert ptr != 0
                    assert torch.equal(_device_bytes(ptr, total).cpu(), src[int(l), int(e)])
        torch.cuda.synchronize()
        tot = M.moe_pool_stats(pool)
        assert (tot.hits, tot.misses) == (hits.sum(), misses.sum())
        assert tot.h2d_bytes == misses.sum() * total
        assert torch.equal(src, before)        # the source is never written
        M.moe_pool_reset(pool)
        assert M.moe_pool_stats(pool).misses == 0
    finally:
        M.moe_pool_destroy(pool)


def test_pooled_decode_equals_resident_decode():
    """OLMoE-shaped layers, 30 of 64 experts resident + 8 spares per layer:
    a chained decode through the pool gives the same bits as the fully
    resident decode (same kernels, same weights, only the table differs)."""
    cfg = MI.PARTIAL
    L, steps = 3, 6
    say("pooled decode L=%d steps=%d" % (L, steps))
    src, devs, total = _pinned_source(cfg, L)
    pool = _make_pool(src, cfg, L, cfg.capacity, cfg.spares, 3, total)
    lays = []
    for l in range(L):
        b = MI.zipf_bias(cfg, l)
        lays.append(MoELayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.g, f16(MI.gen_router(cfg, l)),
                             blob_table(devs[l]), torch.from_numpy(b).to(DEV), device=DEV))
    bufs = [lay.buffers(1) for lay in lays]
    stream = torch.cuda.current_stream()
    misses = 0
    try:
        for s in range(steps):
            x0 = f16(MI.gen_prompt_token(cfg, 0, s))
            xr, xp = x0, x0
            for l, lay in enumerate(lays):
                b = bufs[l]
                # resident reference
                outr = lay.forward(xr, b, residual=xr, out=torch.empty_like(xr))
                ref_idx = b.topk_idx.clone()
                # pooled: route, host ids, prepare, FFN through the pool table
                lay.route_permute(xp, b)
                ids = b.topk_idx.cpu().numpy().reshape(-1).astype(np.int32)
                tab, st = M.moe_pool_prepare(pool, l, ids, ids.size, stream)
                misses += st.misses
                lay.experts(xp, b, table=tab)
                M.moe_pool_retire(pool, l, stream)
                outp = lay.combine(b, residual=xp, out=torch.empty_like(xp))
                torch.cuda.synchronize()
                assert torch.equal(b.topk_idx, ref_idx)
                assert torch.equal(outp.view(torch.int16), outr.view(torch.int16)), (s, l)
                xr, xp = outr, outp
        assert misses > 0      # the run really exercised H2D copies
        assert M.moe_pool_stats(pool).h2d_bytes == misses * total
    finally:
        M.moe_pool_destroy(pool)


def test_native_pooled_layer_equals_resident_decode():
    """moe_pool_layer_forward (route, ids to the host, prepare, FFN, retire,
    combine in one call) gives the bits of the resident decode, and its
    counters match the pool's cumulative ones."""
    cfg = MI.PARTIAL
    L, steps = 3, 6
    say("native pooled layer L=%d steps=%d" % (L, steps))
    src, devs, total = _pinned_source(cfg, L)
    pool = _make_pool(src, cfg, L, cfg.capacity, cfg.spares, 3, total)
    lays = []
    for l in range(L):
        b = MI.zipf_bias(cfg, l)
        lays.append(MoELayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.g, f16(MI.gen_router(cfg, l)),
                             blob_table(devs[l]), torch.from_numpy(b).to(DEV), device=DEV))
    bref = [lay.buffers(1) for lay in lays]
    bpool = [lay.buffers(1) for lay in lays]
    host_ids = torch.empty(cfg.k, dtype=torch.int32, pin_memory=True)
    args = [lay.pool_args(b, host_ids) for lay, b in zip(lays, bpool)]
    stream = torch.cuda.current_stream()
    misses = 0
    uses = np.zeros((L, cfg.E), np.int64)
    miss_map = np.zeros((L, cfg.E), np.int64)
    try:
        for s in range(steps):
            x0 = f16(MI.gen_prompt_token(cfg, 1, s))
            xr, xp = x0, x0
            for l, lay in enumerate(lays):
                outr = lay.forward(xr, bref[l], residual=xr, out=torch.empty_like(xr))
                outp = torch.empty_like(xp)
                a = args[l]
                a.x_f16, a.residual_f16, a.out_f16 = xp.data_ptr(), xp.data_ptr(), outp.data_ptr()
                h0, m0 = M.moe_pool_access_counts(pool, L, cfg.E)
                st = M.moe_pool_layer_forward(pool, l, a, stream)
                misses += st.misses
                # the routed ids the host got (one token: written by the
                # routing kernel into pinned memory) are the device's
                assert np.array_equal(host_ids.numpy(), bpool[l].topk_idx.cpu().numpy().ravel())
                h1, m1 = M.moe_pool_access_counts(pool, L, cfg.E)
                dh, dm = h1 - h0, m1 - m0
                assert dh.sum() == st.hits and dm.sum() == st.misses
                assert np.array_equal(np.flatnonzero(dh[l] + dm[l]), np.sort(host_ids.numpy()))
                uses[l, host_ids.numpy()] += 1
                miss_map += dm
                torch.cuda.synchronize()
                assert torch.equal(bpool[l].topk_idx, bref[l].topk_idx)
                assert torch.equal(outp.view(torch.int16), outr.view(torch.int16)), (s, l)
                xr, xp = outr, outp
        assert misses > 0
        tot = M.moe_pool_stats(pool)
        assert tot.misses == misses and tot.h2d_bytes == misses * total
        # per-(layer, expert) access counts: every routed expert once per call
        h, m = M.moe_pool_access_counts(pool, L, cfg.E)
        assert np.array_equal(h + m, uses) and np.array_equal(m, miss_map)
        assert m.sum() == misses
        M.moe_pool_reset(pool)
        h, m = M.moe_pool_access_counts(pool, L, cfg.E)
        assert not h.any() and not m.any()
    finally:
        M.moe_pool_destroy(pool)


def test_pinned_pool_layer_equals_resident_decode():
    """moe_pool_pin: each layer keeps a fixed set (here the C coldest experts
    of its Zipf bias, so most routed experts miss and the same non-pinned
    expert is copied again token after token).  The native pooled layer still
    gives the resident decode's bits, and hits/misses follow the oracle's
    pinned simulator."""
    cfg = MI.PARTIAL
    L, steps = 2, 6
    say("pinned pooled layer L=%d steps=%d" % (L, steps))
    src, devs, total = _pinned_source(cfg, L)
    pool = _make_pool(src, cfg, L, cfg.capacity, cfg.spares, 3, total)
    lays, pinned = [], []
    for l in range(L):
        b = MI.zipf_bias(cfg, l)
        lays.append(MoELayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.g, f16(MI.gen_router(cfg, l)),
                             blob_table(devs[l]), torch.from_numpy(b).to(DEV), device=DEV))
        pinned.append(np.sort(np.argsort(b, kind="stable")[:cfg.capacity]).astype(np.int32))
    bref = [lay.buffers(1) for lay in lays]
    bpool = [lay.buffers(1) for lay in lays]
    host_ids = torch.empty(cfg.k, dtype=torch.int32, pin_memory=True)
    args = [lay.pool_args(b, host_ids) for lay, b in zip(lays, bpool)]
    stream = torch.cuda.current_stream()
    ev_l, ev_ids, got = [], [], []
    try:
        for l in range(L):
            M.moe_pool_pin(pool, l, pinned[l])
        for s in range(steps):
            x0 = f16(MI.gen_prompt_token(cfg, 2, s))
            xr, xp = x0, x0
            for l, lay in enumerate(lays):
                outr = lay.forward(xr, bref[l], residual=xr, out=torch.empty_like(xr))
                outp = torch.empty_like(xp)
                a = args[l]
                a.x_f16, a.residual_f16, a.out_f16 = xp.data_ptr(), xp.data_ptr(), outp.data_ptr()
                st = M.moe_pool_layer_forward(pool, l, a, stream)
                ev_l.append(l)
                ev_ids.append(host_ids.numpy().copy())
                got.append((st.hits, st.misses, st.evictions))
                torch.cuda.synchronize()
                assert torch.equal(outp.view(torch.int16), outr.view(torch.int16)), (s, l)
                xr, xp = outr, outp
        h, m, _ = O.pool_sim_pinned(L, cfg.E, np.stack(pinned), cfg.k, np.array(ev_l, np.int32),
                                    np.array(ev_ids, np.int32))
        assert [g[:2] for g in got] == list(zip(h.tolist(), m.tolist()))
        assert all(g[2] == 0 for g in got) and m.sum() > h.sum()
    finally:
        M.moe_pool_destroy(pool)
