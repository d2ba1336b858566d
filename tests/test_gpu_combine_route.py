"""moe_combine_route_permute on the GPU: one layer's combine fused with the
next layer's route + permute must give exactly the bits of moe_combine (or
moe_combine_gated) followed by moe_route_permute, in the fused launch (one
decode token, at most 64 experts, fp32 slice partials) and in the cases that
run the two calls, with the decode partials in plain or partial-major column
order; and the routing it produces must equal the oracle's on the combined
activations.  Sources: Horizon RunMap "03 / Arquitetura" (combine,
then the next layer's router) and "08 / Comportamento do modelo" (FP32
routing with explicit roundings)."""
import numpy as np
import pytest
import torch

import int4_weight_only_router_amd as M
from int4_weight_only_router_amd.layer import MoELayer, stack_forward
import moe_inputs as MI
import oracle as O
from tests.gpu_util import DEV, WTOL, f16, make_layer, say

pytestmark = pytest.mark.gpu

KEYS = ("topk_idx", "topk_w", "counts", "offsets", "perm", "inv_perm")


def _np(t):
    return t.detach().cpu().numpy()


def _next_layer(cfg, E=None, k=None, renorm=False, bias=False):
    """A router-only stand-in for layer 1 of cfg (its experts are never run)."""
    E = cfg.E if E is None else E
    k = cfg.k if k is None else k
    c = MI.MoEConfig(cfg.cid, cfg.name, H=cfg.H, E=E, k=k, I=cfg.I, g=cfg.g)
    router = f16(MI.gen_router(c, 1))
    b = None
    if bias:
        b = torch.from_numpy(np.random.default_rng(5).standard_normal(E).astype(np.float32)
                             * np.float32(0.05)).to(DEV)
    table = torch.zeros(E, dtype=torch.int64, device=DEV)
    return MoELayer(cfg.H, cfg.I, E, k, cfg.g, router, table, b, renorm=renorm, device=DEV)


def _run_layer(lay, T, x, partial_order=True):
    b = lay.buffers(T, partial_order=partial_order)
    lay.route_permute(x, b)
    lay.experts(x, b)
    return b


def _snapshot(b, out):
    n = b.T * b.topk_idx.shape[1]
    d = {key: _np(getattr(b, key)).copy() for key in KEYS}
    d["perm"], d["inv_perm"] = d["perm"][:n], d["inv_perm"][:n]
    d["out"] = _np(out).copy()
    return d


def _both(lay, nxt, b, T, x, residual=True):
    """(separate calls, fused call) snapshots for the same layer state."""
    res = x if residual else None
    out_a = torch.empty((T, lay.H), dtype=torch.float16, device=DEV)
    out_b = torch.empty_like(out_a)
    ba, bb = nxt.buffers(T), nxt.buffers(T)
    lay.combine(b, residual=res, out=out_a, x=x)
    nxt.route_permute(out_a, ba)
    lay.combine_route_next(b, nxt, bb, residual=res, out=out_b, x=x)
    torch.cuda.synchronize()
    return _snapshot(ba, out_a), _snapshot(bb, out_b), bb


def _assert_same(a, b, what):
    for key in ("out",) + KEYS:
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), \
            "%s: %s differs" % (what, key)


def _assert_oracle_routing(nxt, snap, cfg_next):
    wr = _np(nxt.router).astype(np.float16)
    bias = None if nxt.bias is None else _np(nxt.bias)
    idx, w, _ = O.route(snap["out"], wr, bias, nxt.k, renorm=bool(nxt.flags & M.MOE_RENORM))
    assert np.array_equal(snap["topk_idx"], idx), "routing differs from the oracle"
    assert np.max(np.abs(snap["topk_w"] - w)) <= WTOL
    counts, offsets, perm, inv = O.permute(idx, nxt.E)
    assert np.array_equal(snap["counts"], counts) and np.array_equal(snap["offsets"], offsets)
    assert np.array_equal(snap["perm"], perm) and np.array_equal(snap["inv_perm"], inv)


CASES = [
    # (config, next E, next k, renorm, bias, residual)
    ("olmoe", None, None, False, False, True),
    ("olmoe", 48, 6, True, True, True),
    ("olmoe", 64, 1, False, True, False),
    ("tiny", None, None, False, False, True),
    ("tiny", 64, 16, True, False, True),
    ("qwen", None, None, False, False, True),       # gated shared expert
    ("h512", 33, 5, False, True, True),
    ("h1024", 64, 8, True, True, True),
]


def _cfg(name):
    if name == "olmoe":
        return MI.OLMOE_DECODE
    if name == "tiny":
        return MI.TINY
    if name == "qwen":
        return MI.QWEN
    if name == "h512":
        return MI.MoEConfig(90, "h512", H=512, E=16, k=4, I=256, g=64)
    return MI.MoEConfig(91, "h1024", H=1024, E=32, k=8, I=512, g=128)


@pytest.mark.parametrize("po", [True, False], ids=["partial_major_y", "plain_y"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-E%s-k%s-r%d-b%d-res%d" % c)
def test_fused_equals_separate_calls(case, po):
    name, En, kn, renorm, bias, residual = case
    cfg = _cfg(name)
    say("combine+route %s" % (case,))
    lay = make_layer(cfg, 0)
    nxt = _next_layer(cfg, En, kn, renorm, bias)
    for s in range(3):
        x = f16(MI.gen_x(cfg, 1, step=s))
        b = _run_layer(lay, 1, x, po)
        assert b.y_dtype == (M.MOE_DTYPE_F32_PM if po else M.MOE_DTYPE_F32) and b.y_slices > 1
        a, f, _ = _both(lay, nxt, b, 1, x, residual)
        _assert_same(a, f, "%s step %d" % (name, s))
        _assert_oracle_routing(nxt, f, cfg)


@pytest.mark.parametrize("T,En", [(2, None), (4, None), (1, 128), (1, 512), (16, None)])
def test_two_call_cases_equal_separate_calls(T, En):
    """Batches above one token, more than 64 experts in the next layer or
    fp16 batched y: the entry point runs the two calls; same bits."""
    cfg = MI.OLMOE_DECODE
    lay = make_layer(cfg, 0)
    nxt = _next_layer(cfg, En, 8 if En else None)
    x = f16(MI.gen_x(cfg, T, step=7))
    b = _run_layer(lay, T, x)
    a, f, _ = _both(lay, nxt, b, T, x)
    _assert_same(a, f, "T=%d E=%s" % (T, En))


def test_routing_arrays_may_be_shared_and_ticket_returns_to_zero():
    """The next layer's routing written into the same arrays the combine reads
    (every read precedes every write), the residual updated in place, and the
    workspace's ticket back at zero after each call."""
    cfg = MI.OLMOE_DECODE
    lay = make_layer(cfg, 0)
    nxt = _next_layer(cfg)
    for s in range(3):
        x = f16(MI.gen_x(cfg, 1, step=20 + s))
        b = _run_layer(lay, 1, x)
        a, _, _ = _both(lay, nxt, b, 1, x)
        xin = x.clone()
        lay.combine_route_next(b, nxt, b, residual=xin, out=xin, x=x)
        torch.cuda.synchronize()
        got = _snapshot(b, xin)
        _assert_same(a, got, "shared arrays step %d" % s)
        assert int(_np(b.perm_ws[:4]).view(np.uint32)[0]) == 0


def test_stack_forward_fused_equals_unfused():
    """Four stacked decode layers: the fused chain (combine + next route in
    one launch) and the plain one give the same bits at every layer."""
    cfg = MI.OLMOE_DECODE
    lays = [make_layer(cfg, l) for l in range(4)]
    outs = {}
    for fuse in (False, True):
        bufs = [lay.buffers(1) for lay in lays]
        acts = [torch.empty((1, cfg.H), dtype=torch.float16, device=DEV) for _ in range(5)]
        acts[0].copy_(f16(MI.gen_x(cfg, 1, step=3)))
        stack_forward(lays, bufs, acts, fuse=fuse)
        torch.cuda.synchronize()
        outs[fuse] = [(_np(a).copy(), _np(bf.topk_idx).copy(), _np(bf.perm).copy())
                      for a, bf in zip(acts[1:], bufs)]
    for l, (u, f) in enumerate(zip(outs[False], outs[True])):
        for i in range(3):
            assert np.array_equal(u[i].view(np.uint8), f[i].view(np.uint8)), (l, i)


def test_rejects_bad_arguments():
    cfg = MI.OLMOE_DECODE
    lay = make_layer(cfg, 0)
    nxt = _next_layer(cfg)
    x = f16(MI.gen_x(cfg, 1, step=0))
    b = _run_layer(lay, 1, x)
    bn = nxt.buffers(1)
    out = torch.empty_like(x)
    with pytest.raises(M.MoEError) as e:   # workspace too small
        M.moe_combine_route_permute(b.y, b.y_dtype, b.y_slices, None, b.topk_w, None, None,
                                    None, x, 1, cfg.H, cfg.k, out, nxt.router, None, nxt.E,
                                    nxt.k, 0, bn.topk_idx, bn.topk_w, bn.counts, bn.offsets,
                                    bn.perm, bn.inv_perm, bn.perm_ws, 256)
    assert e.value.code == M.MOE_ENOMEM
    with pytest.raises(M.MoEError) as e:   # k_next > E
        M.moe_combine_route_permute(b.y, b.y_dtype, b.y_slices, None, b.topk_w, None, None,
                                    None, x, 1, cfg.H, cfg.k, out, nxt.router, None, nxt.E,
                                    nxt.E + 1, 0, bn.topk_idx, bn.topk_w, bn.counts,
                                    bn.offsets, bn.perm, bn.inv_perm, bn.perm_ws,
                                    bn.perm_ws.numel())
    assert e.value.code == M.MOE_EINVAL
    with pytest.raises(M.MoEError) as e:   # a gate without the shared output
        M.moe_combine_route_permute(b.y, b.y_dtype, b.y_slices, None, b.topk_w, None, x,
                                    nxt.router, x, 1, cfg.H, cfg.k, out, nxt.router, None,
                                    nxt.E, nxt.k, 0, bn.topk_idx, bn.topk_w, bn.counts,
                                    bn.offsets, bn.perm, bn.inv_perm, bn.perm_ws,
                                    bn.perm_ws.numel())
    assert e.value.code == M.MOE_EINVAL


SPLIT_CASES = [
    # (config, next-layer renorm, next-layer bias, residual)
    ("olmoe", False, False, True),
    ("olmoe", True, True, True),
    ("tiny", False, True, True),
    ("qwen", False, False, True),       # gated shared expert, 60 experts, top-4
    ("h512", True, False, True),
    ("h1024", False, True, False),
]


@pytest.mark.parametrize("zp", [False, True], ids=["sym", "zero_point"])
@pytest.mark.parametrize("po", [True, False], ids=["partial_major_y", "plain_y"])
@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "%s-r%d-b%d-res%d" % c)
def test_route_in_ffn_equals_fused(case, po, zp):
    """moe_combine_route_partials + moe_expert_ffn_w4a16_routed against
    moe_combine_route_permute + moe_expert_ffn_w4a16: the same out, routing
    arrays and y, bit for bit, over three steps."""
    name, renorm, bias, residual = case
    cfg = _cfg(name)
    fmt = M.MOE_FMT_ZP if zp else M.MOE_FMT_SYM
    say("route in ffn %s po=%d zp=%d" % (case, po, zp))
    lay = make_layer(cfg, 0, fmt=fmt)
    nxt = make_layer(cfg, 1, fmt=fmt)
    if renorm:
        nxt.flags = M.MOE_RENORM
    if bias:
        nxt.bias = torch.from_numpy(np.random.default_rng(6).standard_normal(cfg.E)
                                    .astype(np.float32) * np.float32(0.05)).to(DEV)
    parts = torch.empty(M.moe_logit_partials_bytes() // 4, dtype=torch.float32, device=DEV)
    for s in range(3):
        x = f16(MI.gen_x(cfg, 1, step=20 + s))
        b = _run_layer(lay, 1, x, po)
        assert lay.split_route_ok(b, nxt)
        res = x if residual else None
        out_a = torch.empty((1, cfg.H), dtype=torch.float16, device=DEV)
        out_b = torch.empty_like(out_a)
        ba, bb = nxt.buffers(1, partial_order=po), nxt.buffers(1, partial_order=po)
        bb.y.fill_(-7.0)
        lay.combine_route_next(b, nxt, ba, residual=res, out=out_a, x=x)
        nxt.experts(out_a, ba)
        lay.combine_partials_next(b, nxt, parts, residual=res, out=out_b, x=x)
        nxt.experts_routed(out_b, bb, parts)
        torch.cuda.synchronize()
        a, f = _snapshot(ba, out_a), _snapshot(bb, out_b)
        _assert_same(a, f, "%s step %d" % (name, s))
        assert np.array_equal(_np(ba.y).view(np.uint8), _np(bb.y).view(np.uint8)), \
            "%s step %d: y differs" % (name, s)
        _assert_oracle_routing(nxt, f, cfg)


SPLIT_NEXT = [
    # (config, next E, next k, renorm, bias): next layers of other expert counts
    ("olmoe", 37, 5, False, True),
    ("olmoe", 64, 16, True, False),
    ("olmoe", 48, 1, False, False),
    ("h512", 33, 5, True, True),
    ("h1024", 9, 8, False, True),
]


@pytest.mark.parametrize("case", SPLIT_NEXT, ids=lambda c: "%s-E%d-k%d-r%d-b%d" % c)
def test_route_in_ffn_other_expert_counts(case):
    """The split form against the fused one when the next layer has another
    expert count and top-k (E not a multiple of 8, k = 1 and 16, k close to
    E): out, routing arrays and y bit for bit, routing against the oracle."""
    name, En, kn, renorm, bias = case
    cfg = _cfg(name)
    cn = MI.MoEConfig(cfg.cid + 40 + En, "%s-next-E%d" % (name, En), H=cfg.H, E=En, k=kn,
                      I=cfg.I, g=cfg.g)
    say("route in ffn, next layer %s" % (case,))
    lay = make_layer(cfg, 0)
    nxt = make_layer(cn, 1)
    if renorm:
        nxt.flags = M.MOE_RENORM
    if bias:
        nxt.bias = torch.from_numpy(np.random.default_rng(7).standard_normal(En)
                                    .astype(np.float32) * np.float32(0.05)).to(DEV)
    parts = torch.empty(M.moe_logit_partials_bytes() // 4, dtype=torch.float32, device=DEV)
    for s in range(2):
        x = f16(MI.gen_x(cfg, 1, step=40 + s))
        b = _run_layer(lay, 1, x)
        assert lay.split_route_ok(b, nxt)
        out_a = torch.empty((1, cfg.H), dtype=torch.float16, device=DEV)
        out_b = torch.empty_like(out_a)
        ba, bb = nxt.buffers(1), nxt.buffers(1)
        bb.y.fill_(-7.0)
        lay.combine_route_next(b, nxt, ba, residual=x, out=out_a, x=x)
        nxt.experts(out_a, ba)
        lay.combine_partials_next(b, nxt, parts, residual=x, out=out_b, x=x)
        nxt.experts_routed(out_b, bb, parts)
        torch.cuda.synchronize()
        a, f = _snapshot(ba, out_a), _snapshot(bb, out_b)
        _assert_same(a, f, "%s step %d" % (case, s))
        assert np.array_equal(_np(ba.y).view(np.uint8), _np(bb.y).view(np.uint8)), \
            "%s step %d: y differs" % (case, s)
        _assert_oracle_routing(nxt, f, cn)


@pytest.mark.parametrize("zp", [False, True], ids=["sym", "zero_point"])
@pytest.mark.parametrize("name,renorm,bias", [("olmoe", False, False), ("olmoe", True, True),
                                              ("tiny", False, True), ("qwen", False, False),
                                              ("h512", True, True), ("h1024", False, True)])
def test_first_layer_partials_equal_route_permute(name, renorm, bias, zp):
    """moe_logit_partials + moe_expert_ffn_w4a16_routed against
    moe_route_permute + moe_expert_ffn_w4a16 on one input row: routing arrays
    and y bit for bit, routing against the oracle."""
    cfg = _cfg(name)
    say("first-layer partials %s renorm=%d bias=%d zp=%d" % (name, renorm, bias, zp))
    lay = make_layer(cfg, 1, fmt=M.MOE_FMT_ZP if zp else M.MOE_FMT_SYM)
    if renorm:
        lay.flags = M.MOE_RENORM
    if bias:
        lay.bias = torch.from_numpy(np.random.default_rng(8).standard_normal(cfg.E)
                                    .astype(np.float32) * np.float32(0.05)).to(DEV)
    parts = torch.empty(M.moe_logit_partials_bytes() // 4, dtype=torch.float32, device=DEV)
    for s in range(3):
        x = f16(MI.gen_x(cfg, 1, step=60 + s))
        ba, bb = lay.buffers(1), lay.buffers(1)
        assert lay.route_from_partials_ok(bb)
        bb.y.fill_(-7.0)
        lay.route_permute(x, ba)
        lay.experts(x, ba)
        lay.logit_partials(x, parts)
        lay.experts_routed(x, bb, parts)
        torch.cuda.synchronize()
        a, f = _snapshot(ba, x), _snapshot(bb, x)
        _assert_same(a, f, "%s step %d" % (name, s))
        assert np.array_equal(_np(ba.y).view(np.uint8), _np(bb.y).view(np.uint8)), \
            "%s step %d: y differs" % (name, s)
        _assert_oracle_routing(lay, f, cfg)


def test_route_in_ffn_rejects_other_shapes():
    """Two tokens, more than 64 experts or a batched y: MOE_EUNSUPPORTED before
    any launch."""
    cfg = MI.OLMOE_DECODE
    lay = make_layer(cfg, 0)
    parts = torch.empty(M.moe_logit_partials_bytes() // 4, dtype=torch.float32, device=DEV)
    b2 = lay.buffers(2)
    with pytest.raises(M.MoEError) as ei:
        M.moe_expert_ffn_w4a16_routed(b2.out, parts, None, cfg.E, cfg.k, 0, b2.topk_idx,
                                      b2.topk_w, b2.counts, b2.offsets, b2.perm, b2.inv_perm,
                                      lay.table, 2, cfg.H, cfg.I, cfg.g, b2.regime, b2.y,
                                      b2.y_dtype, b2.y_slices)
    assert ei.value.code == M.MOE_EUNSUPPORTED
    nxt = _next_layer(cfg, 128, 8)
    b = lay.buffers(1)
    with pytest.raises(M.MoEError) as ei:
        M.moe_combine_route_partials(b.y, b.y_dtype, b.y_slices, None, b.topk_w, None, None,
                                     None, None, 1, cfg.H, cfg.k, b.out, nxt.router, 128, parts)
    assert ei.value.code == M.MOE_EUNSUPPORTED
