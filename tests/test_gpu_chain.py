"""Stacked layers and layer-level special cases on the GPU, against the oracle.

Chained runs are checked layer by layer with teacher forcing: each layer's
oracle takes, as its input and residual, the exact fp16 activations the GPU
layer received, and must reproduce the GPU's routing bit for bit (indices,
counts, offsets, permutation, inverse) and its output within the stated
tolerance.  The free-running divergence of the oracle's own chain from the
GPU's (routing flips, output drift) is printed, not gated.

Workloads: the 16-layer OLMoE-shaped decode chain (hidden 2048, 64 experts,
top-8, I = 1024, g = 128, one token per step, x_{l+1} = fp16(x_l + MoE_l(x_l)))
replayed as one captured graph per step, as the benchmark times it; and the
same chain with 30 of 64 experts per layer in the slot pool (Zipf(1.0) router
bias), one native pooled-layer call per layer, whose per-call pool counters
must also equal the oracle's residency simulator.

Special cases that reduce to closed forms: every expert identical (the output
is the residual plus the sum of the token's routing weights times one dense
SwiGLU FFN) and zero activations (the output equals the residual bit for bit,
the routing is experts 0..k-1 with weight 1/E each)."""
import numpy as np
import pytest
import torch

import int4_weight_only_router_amd as M
from int4_weight_only_router_amd.layer import MoELayer, blob_table, stack_forward
import moe_inputs as MI
import oracle as O
from tests.gpu_util import (DEV, WTOL, OracleBlobs, check_close, device_experts, f16, make_layer,
                            say)

pytestmark = pytest.mark.gpu

STEPS = 3


def _np(t):
    return t.detach().cpu().numpy()


def _layers(cfg, L):
    """L device-resident layers of cfg (library quantiser and prepack)."""
    lays = []
    for l in range(L):
        say("build %s layer %d" % (cfg.name, l))
        dev, _ = device_experts(cfg, l)
        b = MI.zipf_bias(cfg, l)
        lay = MoELayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.g, f16(MI.gen_router(cfg, l)),
                       blob_table(dev), None if b is None else torch.from_numpy(b).to(DEV),
                       device=DEV)
        lay._blobs = dev
        lays.append(lay)
    return lays


def _check_layer(cfg, l, obl, rec, what):
    """Teacher-forced oracle of layer l on the GPU layer's own input."""
    x = rec["x"]
    wr = MI.gen_router(cfg, l)
    bias = MI.zipf_bias(cfg, l)
    idx, _, _ = O.route(x, wr, bias, cfg.k)
    ref = O.moe_layer(x, wr, obl.get(np.unique(idx)), cfg.H, cfg.I, cfg.E, cfg.k, cfg.g,
                      bias=bias, residual=x)
    for key in ("idx", "counts", "offsets", "perm", "inv_perm"):
        assert np.array_equal(rec[key], ref[key]), "%s: %s differs" % (what, key)
    assert np.max(np.abs(rec["w"] - ref["w"])) <= WTOL, what
    return check_close(rec["out"].astype(np.float64), ref["out_f64"], what)


def _record(x, b, out, T, k):
    n = T * k
    return dict(x=_np(x).copy(), idx=_np(b.topk_idx).copy(), w=_np(b.topk_w).copy(),
                counts=_np(b.counts).copy(), offsets=_np(b.offsets).copy(),
                perm=_np(b.perm)[:n].copy(), inv_perm=_np(b.inv_perm)[:n].copy(),
                out=_np(out).copy())


def _free_running(cfg, L, x0, obls):
    """The oracle's own chain from x0 (no teacher forcing): final output and
    the routed sets of every layer."""
    x = x0
    sets = []
    for l in range(L):
        wr = MI.gen_router(cfg, l)
        bias = MI.zipf_bias(cfg, l)
        idx, _, _ = O.route(x, wr, bias, cfg.k)
        ref = O.moe_layer(x, wr, obls[l].get(np.unique(idx)), cfg.H, cfg.I, cfg.E, cfg.k,
                          cfg.g, bias=bias, residual=x)
        sets.append(ref["idx"])
        x = ref["out"]
    return x, sets


@pytest.mark.parametrize("fuse", ["three_calls", "combine_route_fused", "route_in_ffn"])
def test_decode_chain_16_layers_teacher_forced(fuse):
    """The benchmark's workload and launch configuration: 16 stacked decode
    layers captured in one graph, replayed once per step (fresh x0 each
    step); every layer of every step against the oracle.  combine_route_fused:
    each layer's combine runs with the next layer's route + permute in one
    launch; route_in_ffn: the combine hands on only the next layer's logit
    partials and that layer's expert launch routes from them."""
    cfg = MI.OLMOE_DECODE
    L = cfg.layers
    lays = _layers(cfg, L)
    bufs = [lay.buffers(1) for lay in lays]
    assert bufs[0].regime & ~(M.MOE_Y_TOKEN_ORDER | M.MOE_Y_PARTIAL_ORDER) == \
        M.MOE_REGIME_DECODE
    acts = [torch.empty((1, cfg.H), dtype=torch.float16, device=DEV) for _ in range(L + 1)]
    parts = torch.empty(M.moe_logit_partials_bytes() // 4, dtype=torch.float32, device=DEV)

    def step():
        if fuse != "three_calls":
            stack_forward(lays, bufs, acts, parts=parts if fuse == "route_in_ffn" else None)
            return
        for l, lay in enumerate(lays):
            lay.forward(acts[l], bufs[l], residual=acts[l], out=acts[l + 1])

    acts[0].copy_(f16(MI.gen_x(cfg, 1, step=100)))
    step()                                  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    obls = [OracleBlobs(cfg, l) for l in range(L)]
    worst = 0.0
    for s in range(STEPS):
        x0 = MI.gen_x(cfg, 1, step=s)
        acts[0].copy_(f16(x0))
        say("decode chain step %d: graph replay" % s)
        g.replay()
        torch.cuda.synchronize()
        recs = [_record(acts[l], bufs[l], acts[l + 1], 1, cfg.k) for l in range(L)]
        for l in range(L):
            mx, _ = _check_layer(cfg, l, obls[l], recs[l], "step %d layer %d" % (s, l))
            worst = max(worst, mx)
        fin, sets = _free_running(cfg, L, x0, obls)
        flips = sum(int(not np.array_equal(sets[l], recs[l]["idx"])) for l in range(L))
        drift = float(np.max(np.abs(fin.astype(np.float64) - recs[-1]["out"].astype(np.float64))))
        say("step %d: teacher-forced worst max|d| %.3g; free-running: %d of %d layers route "
            "differently, final max|d| %.3g (reported, not gated)" % (s, worst, flips, L, drift))


def test_pooled_chain_16_layers_teacher_forced():
    """Partial residency: 16 layers, 30 of 64 experts resident per layer plus
    8 spares, the INT4 source in pinned host memory; per token and layer one
    moe_pool_layer_forward call.  Every layer against the oracle (teacher
    forced) and every call's hits/misses/evictions against the simulator."""
    cfg = MI.PARTIAL
    L = cfg.layers
    _, total = M.moe_blob_layout(cfg.H, cfg.I, cfg.g)
    src = torch.empty((L, cfg.E, total), dtype=torch.uint8, pin_memory=True)
    lays = []
    for l in range(L):
        say("build %s layer %d (pinned source)" % (cfg.name, l))
        dev, _ = device_experts(cfg, l)
        src[l].copy_(dev)
        torch.cuda.synchronize()
        b = MI.zipf_bias(cfg, l)
        lay = MoELayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.g, f16(MI.gen_router(cfg, l)),
                       blob_table(dev), torch.from_numpy(b).to(DEV), device=DEV)
        lay._blobs = dev        # the pooled calls read the pool's table, not this one
        lays.append(lay)
    ptrs = [src[l, e].data_ptr() for l in range(L) for e in range(cfg.E)]
    pc = M.PoolConfig(layers=L, experts=cfg.E, topk=cfg.k, capacity=cfg.capacity,
                      spares=cfg.spares, decay_shift=3, expert_bytes=total)
    pool = M.moe_pool_create(pc, ptrs)
    bufs = [lay.buffers(1) for lay in lays]
    host_ids = torch.empty(cfg.k, dtype=torch.int32, pin_memory=True)
    args = [lay.pool_args(b, host_ids) for lay, b in zip(lays, bufs)]
    acts = [torch.empty((1, cfg.H), dtype=torch.float16, device=DEV) for _ in range(L + 1)]
    stream = torch.cuda.current_stream()
    obls = [OracleBlobs(cfg, l) for l in range(L)]
    ev_l, ev_ids, got = [], [], []
    try:
        for s in range(STEPS):
            acts[0].copy_(f16(MI.gen_prompt_token(cfg, 0, s)))
            say("pooled chain step %d" % s)
            recs = []
            for l in range(L):
                a = args[l]
                a.x_f16 = a.residual_f16 = acts[l].data_ptr()
                a.out_f16 = acts[l + 1].data_ptr()
                st = M.moe_pool_layer_forward(pool, l, a, stream)
                torch.cuda.synchronize()
                ev_l.append(l)
                ev_ids.append(host_ids.numpy().copy())
                got.append((st.hits, st.misses, st.evictions, st.h2d_bytes))
                recs.append(_record(acts[l], bufs[l], acts[l + 1], 1, cfg.k))
            for l in range(L):
                _check_layer(cfg, l, obls[l], recs[l], "pooled step %d layer %d" % (s, l))
        h, m, _, _ = O.pool_sim(L, cfg.E, cfg.capacity, 3, cfg.k, np.array(ev_l, np.int32),
                                np.array(ev_ids, np.int32))
        assert [g_[:3] for g_ in got] == list(zip(h.tolist(), m.tolist(), m.tolist()))
        assert [g_[3] for g_ in got] == (m.astype(np.int64) * total).tolist()
        assert m.sum() > 0                  # copies really happened
        say("pooled chain: %d misses over %d calls" % (int(m.sum()), len(got)))
    finally:
        M.moe_pool_destroy(pool)


# ------------------------------------------------ layer-level special cases

CASES = [(1, M.MOE_REGIME_DECODE), (3, M.MOE_REGIME_DECODE), (16, M.MOE_REGIME_SMALL),
         (300, M.MOE_REGIME_BATCHED)]


@pytest.mark.parametrize("T,regime", CASES)
def test_layer_zero_input_gives_residual(T, regime):
    """x = 0: every logit is exactly 0, so the routing is experts 0..k-1 (the
    lower-index tie-break) with weight 1/E; the routed and shared FFNs of a
    zero vector are exactly zero, so the output is the residual, bit for bit."""
    cfg = MI.E512
    lay = make_layer(cfg, 0)
    lay.bias = None
    say("zero input %s T=%d regime=%d" % (cfg.name, T, regime))
    x = np.zeros((T, cfg.H), np.float16)
    res = MI.gen_residual(cfg, T)
    b = lay.buffers(T, regime)
    out = lay.forward(f16(x), b, residual=f16(res))
    torch.cuda.synchronize()
    assert np.array_equal(_np(b.topk_idx), np.tile(np.arange(cfg.k, dtype=np.int32), (T, 1)))
    assert np.max(np.abs(_np(b.topk_w) - 1.0 / cfg.E)) <= WTOL
    assert np.array_equal(_np(out).view(np.uint16), res.view(np.uint16))
    # the oracle agrees
    ref = O.moe_layer(x, MI.gen_router(cfg, 0), OracleBlobs(cfg, 0).get(range(cfg.k)), cfg.H,
                      cfg.I, cfg.E, cfg.k, cfg.g, shared=MI.gen_shared(cfg), residual=res)
    assert np.array_equal(ref["out"].view(np.uint16), res.view(np.uint16))


@pytest.mark.parametrize("T,regime", CASES)
def test_layer_all_experts_identical(T, regime):
    """Every table entry points at the same expert blob: the layer output is
    residual + (sum_j w[t,j]) * FFN(x_t), the FFN evaluated once, densely, from
    the dequantised matrices (a plain fp64 SwiGLU, written here)."""
    cfg = MI.OLMOE_DECODE
    lay = make_layer(cfg, 0, shared=False)
    base = lay._blobs[3]
    lay.table = torch.full((cfg.E,), base.data_ptr(), dtype=torch.int64, device=DEV)
    say("identical experts %s T=%d regime=%d" % (cfg.name, T, regime))
    x = MI.gen_x(cfg, T, step=11)
    res = MI.gen_residual(cfg, T)
    b = lay.buffers(T, regime)
    out = lay.forward(f16(x), b, residual=f16(res))
    torch.cuda.synchronize()
    blob = OracleBlobs(cfg, 0).get([3])[3]
    ref = O.moe_layer(x, MI.gen_router(cfg, 0), [blob] * cfg.E, cfg.H, cfg.I, cfg.E, cfg.k,
                      cfg.g, residual=res)
    assert np.array_equal(_np(b.topk_idx), ref["idx"])
    got = _np(out).astype(np.float64)
    check_close(got, ref["out_f64"], "identical experts vs oracle T=%d" % T)
    gq, uq, dq, gs, us, ds = O.blob_sections(blob, cfg.H, cfg.I, cfg.g)
    Wg, Wu, Wd = (O.dequant_rows(gq, gs, cfg.g), O.dequant_rows(uq, us, cfg.g),
                  O.dequant_rows(dq, ds, cfg.g))
    xv = x.astype(np.float64)
    a, u = xv @ Wg.T, xv @ Wu.T
    ffn = ((a / (1.0 + np.exp(-a))) * u) @ Wd.T
    wsum = _np(b.topk_w).astype(np.float64).sum(axis=1, keepdims=True)
    closed = res.astype(np.float64) + wsum * ffn
    check_close(got, closed, "identical experts vs closed form T=%d" % T)
