"""GPU parity: every entry point of libmoe_w4a16 against the CPU oracle on
the same seeded inputs.  Integer results (quantised codes, routing indices,
counts, offsets, permutations) must match bit for bit; floating results
within max|d| <= 2e-2 and relative L2 <= 1e-2 (routing weights within 1e-5).
The routed FFN is compared on every row at every size (the oracle spreads
rows over threads); whole layers on every token up to 512 tokens and, at
4096, on the tokens of the first and last row of every expert bucket (tile
edges) plus seeded random tokens."""
import numpy as np
import pytest
import torch

import int4_weight_only_router_amd as M
from int4_weight_only_router_amd.layer import MoELayer, blob_table
import moe_inputs as MI
import oracle as O
from tests.gpu_util import (DEV, WTOL, OracleBlobs, check_close, device_experts, f16,
                            make_layer, pm_positions, sample_rows, say, y_plain)
from tests.layout_util import numpy_prepack as _numpy_prepack

pytestmark = pytest.mark.gpu

# group size 32 and an intermediate size (192) that leaves the last 256-column
# tile of the fused gate/up matrix half empty
G32 = MI.MoEConfig(91, "g32_i192", H=512, E=16, k=4, I=192, g=32)
# fused router above 128 experts with a ragged last 64-expert block, up to the
# largest expert count and k
E1000 = MI.MoEConfig(94, "h256_e1000_k16", H=256, E=1000, k=16, I=128, g=64, zipf_s=1.1)
E200 = MI.MoEConfig(95, "h512_e200_k3", H=512, E=200, k=3, I=128, g=64)


def _np(t):
    return t.detach().cpu().numpy()


# ------------------------------------------------------------- quantiser

@pytest.mark.parametrize("cfg", [MI.TINY, MI.OLMOE_DECODE, MI.E512], ids=lambda c: c.name)
def test_quantize_bit_exact(cfg):
    say("quantize %s" % cfg.name)
    _, canon = device_experts(cfg, 0, experts=[0, 1, cfg.E - 1])
    ob = OracleBlobs(cfg, 0).get([0, 1, cfg.E - 1])
    for e in (0, 1, cfg.E - 1):
        assert np.array_equal(_np(canon[e]), ob[e]), "expert %d blob differs" % e


def test_prepack_layout_and_round_trip():
    cfg = MI.TINY
    say("prepack round trip")
    dev, canon = device_experts(cfg, 0, experts=[0, 3])
    for e in (0, 3):
        ref = _numpy_prepack(_np(canon[e]), cfg.H, cfg.I, cfg.g)
        assert np.array_equal(_np(dev[e]), ref)
        host = np.empty_like(ref)   # the host bijection gives the same bytes
        M.moe_prepack_expert_host(_np(canon[e]), cfg.H, cfg.I, cfg.g, M.MOE_FMT_SYM, host)
        assert np.array_equal(host, ref)
    back = torch.empty_like(dev)
    M.moe_unpack_experts(dev, cfg.E, cfg.H, cfg.I, cfg.g, back)
    torch.cuda.synchronize()
    for e in (0, 3):
        assert np.array_equal(_np(back[e]), _np(canon[e]))


# ---------------------------------------------------------------- router

def _route_gpu(x, wr, bias, T, H, E, k, flags=0):
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    wsb = M.moe_route_workspace_bytes(T, E)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=DEV)
    M.moe_route(x, wr, bias, T, H, E, k, flags, idx, w, ws, wsb)
    torch.cuda.synchronize()
    return _np(idx), _np(w)


@pytest.mark.parametrize("cfg,T,renorm", [
    (MI.TINY, 16, False), (MI.TINY, 16, True), (MI.OLMOE_DECODE, 1, False),
    (MI.OLMOE_DECODE, 64, False), (MI.OLMOE_DECODE, 512, False),
    (MI.OLMOE_DECODE, 4096, False), (MI.E512, 1, False), (MI.E512, 256, False),
    (MI.E512, 4096, False), (MI.OLMOE_DECODE, 67, False)],
    ids=lambda v: getattr(v, "name", str(v)))
def test_route_bit_exact(cfg, T, renorm):
    say("route %s T=%d renorm=%d" % (cfg.name, T, renorm))
    x = MI.gen_x(cfg, T)
    wr = MI.gen_router(cfg)
    b = MI.zipf_bias(cfg)
    idx, w = _route_gpu(f16(x), f16(wr), None if b is None else torch.from_numpy(b).to(DEV),
                        T, cfg.H, cfg.E, cfg.k, M.MOE_RENORM if renorm else 0)
    toks = np.arange(T) if T <= 512 else np.random.default_rng(T).choice(T, 256, replace=False)
    oi, ow, _ = O.route(x[toks], wr, b, cfg.k, renorm)
    assert np.array_equal(idx[toks], oi)
    assert np.max(np.abs(w[toks] - ow)) <= WTOL


@pytest.mark.parametrize("cfg,T", [(MI.OLMOE_DECODE, 1), (MI.OLMOE_DECODE, 3),
                                   (MI.OLMOE_DECODE, 8), (MI.OLMOE_DECODE, 9), (MI.E512, 1),
                                   (MI.E512, 5), (MI.TINY, 16), (MI.E512, 70), (E1000, 1),
                                   (E1000, 4), (E200, 2), (E200, 3)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_route_permute_fused_bit_exact(cfg, T):
    say("route_permute %s T=%d" % (cfg.name, T))
    x = MI.gen_x(cfg, T, step=7)
    wr = MI.gen_router(cfg)
    b = MI.zipf_bias(cfg)
    n = T * cfg.k
    idx = torch.empty((T, cfg.k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, cfg.k), dtype=torch.float32, device=DEV)
    counts = torch.full((cfg.E,), -7, dtype=torch.int32, device=DEV)
    offsets = torch.full((cfg.E + 1,), -7, dtype=torch.int32, device=DEV)
    perm = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    inv = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    wsb = M.moe_route_permute_workspace_bytes(T, cfg.k, cfg.E)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=DEV)
    for rep in range(2):   # the workspace is reusable: the second call must agree
      M.moe_route_permute(f16(x), f16(wr), None if b is None else torch.from_numpy(b).to(DEV),
                          T, cfg.H, cfg.E, cfg.k, 0, idx, w, counts, offsets, perm, inv, ws, wsb)
      torch.cuda.synchronize()
      oi, ow, _ = O.route(x, wr, b, cfg.k)
      assert np.array_equal(_np(idx), oi)
      assert np.max(np.abs(_np(w) - ow)) <= WTOL
      for got, ref, name in zip((counts, offsets, perm, inv), O.permute(oi, cfg.E),
                                ("counts", "offsets", "perm", "inv_perm")):
          assert np.array_equal(_np(got), ref), name
      assert int(_np(ws[:4].view(torch.int32))[0]) == 0   # ticket zero after either path


@pytest.mark.parametrize("cfg,Ts", [(MI.OLMOE_DECODE, (3, 40, 3, 5, 6, 1)),
                                    (MI.E512, (2, 9, 2, 4, 5, 1))],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_route_permute_one_workspace_across_batch_sizes(cfg, Ts):
    """One workspace (sized for the largest T) serves batches on both sides
    of the fused/two-launch boundary, in any order."""
    say("route_permute shared ws %s" % cfg.name)
    wr = f16(MI.gen_router(cfg))
    b = MI.zipf_bias(cfg)
    bias = None if b is None else torch.from_numpy(b).to(DEV)
    wsb = max(M.moe_route_permute_workspace_bytes(T, cfg.k, cfg.E) for T in Ts)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    for i, T in enumerate(Ts):
        x = MI.gen_x(cfg, T, step=20 + i)
        n = T * cfg.k
        idx = torch.empty((T, cfg.k), dtype=torch.int32, device=DEV)
        w = torch.empty((T, cfg.k), dtype=torch.float32, device=DEV)
        counts = torch.empty(cfg.E, dtype=torch.int32, device=DEV)
        offsets = torch.empty(cfg.E + 1, dtype=torch.int32, device=DEV)
        perm = torch.empty(n, dtype=torch.int32, device=DEV)
        inv = torch.empty(n, dtype=torch.int32, device=DEV)
        M.moe_route_permute(f16(x), wr, bias, T, cfg.H, cfg.E, cfg.k, 0, idx, w, counts, offsets,
                            perm, inv, ws, wsb)
        torch.cuda.synchronize()
        oi, ow, _ = O.route(x, MI.gen_router(cfg), b, cfg.k)
        assert np.array_equal(_np(idx), oi), T
        for got, ref in zip((counts, offsets, perm, inv), O.permute(oi, cfg.E)):
            assert np.array_equal(_np(got), ref), T
        assert int(_np(ws[:4].view(torch.int32))[0]) == 0


H1024 = MI.MoEConfig(88, "h1024_e64", H=1024, E=64, k=6, I=128, g=64)


# the fused launch (one token to a few), the one-workgroup router and the
# register-tiled logits kernel up to 8200 tokens: H = 256, 512, 1024, 2048;
# ragged T and E tails
@pytest.mark.parametrize("cfg,T", [(MI.OLMOE_DECODE, 1), (MI.OLMOE_DECODE, 5), (MI.E512, 1),
                                   (MI.E512, 7), (MI.TINY, 16), (MI.OLMOE_DECODE, 64),
                                   (MI.E512, 300), (MI.E512, 4096), (MI.OLMOE_DECODE, 4096),
                                   (MI.QWEN, 4100), (MI.TINY, 8200), (E1000, 300), (E200, 1300),
                                   (H1024, 4096)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_router_logits_pinned_order(cfg, T):
    """The logits the router kernels leave in their workspace equal the
    oracle's pinned-order fp32 logits bit for bit (chunk c of 8 elements into
    partial c mod 64 by single-rounding FMAs, xor butterfly, then the bias)."""
    say("logits %s T=%d" % (cfg.name, T))
    x = MI.gen_x(cfg, T, step=11)
    wr = MI.gen_router(cfg)
    b = MI.zipf_bias(cfg)
    n = T * cfg.k
    idx = torch.empty((T, cfg.k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, cfg.k), dtype=torch.float32, device=DEV)
    counts = torch.empty(cfg.E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(cfg.E + 1, dtype=torch.int32, device=DEV)
    perm = torch.empty(n, dtype=torch.int32, device=DEV)
    inv = torch.empty(n, dtype=torch.int32, device=DEV)
    wsb = M.moe_route_permute_workspace_bytes(T, cfg.k, cfg.E)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    M.moe_route_permute(f16(x), f16(wr), None if b is None else torch.from_numpy(b).to(DEV),
                        T, cfg.H, cfg.E, cfg.k, 0, idx, w, counts, offsets, perm, inv, ws, wsb)
    torch.cuda.synchronize()
    # either path keeps the fused launch's 256-byte ticket first, then the
    # T x E logits
    off = 256
    got = _np(ws[off:off + T * cfg.E * 4].view(torch.float32)).reshape(T, cfg.E)
    _, _, ref = O.route(x, wr, b, cfg.k)
    assert np.array_equal(got.view(np.int32), ref.view(np.int32))


def test_route_ties_go_to_lower_index():
    cfg = MI.OLMOE_DECODE
    say("route ties")
    T = 8
    x = MI.gen_x(cfg, T)
    x[0] = 0.0                                  # all logits equal -> experts 0..k-1
    wr = MI.gen_router(cfg)
    wr[40] = wr[3]                              # duplicated rows -> exact ties
    wr[17] = wr[3]
    wr[63] = wr[9]
    idx, w = _route_gpu(f16(x), f16(wr), None, T, cfg.H, cfg.E, cfg.k)
    oi, ow, _ = O.route(x, wr, None, cfg.k)
    assert np.array_equal(idx, oi)
    assert np.array_equal(idx[0], np.arange(cfg.k))
    assert np.max(np.abs(w - ow)) <= WTOL


@pytest.mark.parametrize("T,fused", [(1, True), (3, True), (8, False), (64, False)])
def test_route_ties_512_experts(T, fused):
    """The 512-expert selection (k rounds of a wave-wide key maximum) keeps
    the lower expert index first on exact ties, also across lanes and key
    slots, on the fused (route + sort) and the separate router paths."""
    cfg = MI.E512
    say("route ties E=512 T=%d fused=%d" % (T, fused))
    x = MI.gen_x(cfg, T)
    x[0] = 0.0                                  # all 512 logits equal -> experts 0..k-1
    wr = MI.gen_router(cfg)
    wr[400] = wr[3]                             # duplicated rows -> exact ties in other
    wr[511] = wr[3]                             # lanes and key slots
    wr[64] = wr[9]
    wr[137] = wr[200]
    if fused:
        n = T * cfg.k
        idx_t = torch.empty((T, cfg.k), dtype=torch.int32, device=DEV)
        w_t = torch.empty((T, cfg.k), dtype=torch.float32, device=DEV)
        counts = torch.empty(cfg.E, dtype=torch.int32, device=DEV)
        offsets = torch.empty(cfg.E + 1, dtype=torch.int32, device=DEV)
        perm = torch.empty(n, dtype=torch.int32, device=DEV)
        inv = torch.empty(n, dtype=torch.int32, device=DEV)
        wsb = M.moe_route_permute_workspace_bytes(T, cfg.k, cfg.E)
        ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
        M.moe_route_permute(f16(x), f16(wr), None, T, cfg.H, cfg.E, cfg.k, 0, idx_t, w_t, counts,
                            offsets, perm, inv, ws, wsb)
        torch.cuda.synchronize()
        idx, w = _np(idx_t), _np(w_t)
        oi, ow, _ = O.route(x, wr, None, cfg.k)
        c_ref, o_ref, p_ref, _ = O.permute(oi, cfg.E)
        assert np.array_equal(_np(offsets), o_ref) and np.array_equal(_np(perm), p_ref[:n])
    else:
        idx, w = _route_gpu(f16(x), f16(wr), None, T, cfg.H, cfg.E, cfg.k)
        oi, ow, _ = O.route(x, wr, None, cfg.k)
    assert np.array_equal(idx, oi)
    assert np.array_equal(idx[0], np.arange(cfg.k))
    assert np.max(np.abs(w - ow)) <= WTOL


# ----------------------------------------------------------- permutation

def _permute_gpu(idx_np, E):
    T, k = idx_np.shape
    n = T * k
    idx = torch.from_numpy(idx_np).to(DEV)
    counts = torch.full((E,), -7, dtype=torch.int32, device=DEV)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    perm = torch.full((max(n, 1),), -7, dtype=torch.int32, device=DEV)
    inv = torch.full((max(n, 1),), -7, dtype=torch.int32, device=DEV)
    wsb = M.moe_permute_workspace_bytes(T, k, E)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=DEV)
    M.moe_permute(idx, T, k, E, counts, offsets, perm, inv, ws, wsb)
    torch.cuda.synchronize()
    return _np(counts), _np(offsets), _np(perm)[:n], _np(inv)[:n]


@pytest.mark.parametrize("T,k,E,skew", [(1, 8, 64, 0), (16, 2, 8, 0), (64, 8, 64, 0),
                                        (512, 8, 64, 0), (513, 8, 64, 0), (4096, 8, 64, 0),
                                        (4096, 10, 512, 1.1), (300, 16, 1024, 1.0),
                                        (1024, 10, 512, 1.1), (1025, 10, 512, 1.1),
                                        (640, 16, 1024, 0), (1, 1, 1, 0), (0, 8, 64, 0)])
def test_permute_bit_exact(T, k, E, skew):
    """Every sort path: one wave (T*k <= 512), one workgroup (up to 10240
    elements, E <= 1024; 10240 itself and 10250 either side of the limit, and
    E = 1024 with its 64 KB of per-wave histograms), chunked launches above."""
    say("permute T=%d k=%d E=%d" % (T, k, E))
    rng = np.random.default_rng(T * 7 + E)
    p = None
    if skew:
        p = np.arange(1, E + 1, dtype=np.float64) ** -skew
        p /= p.sum()
    idx = np.array([rng.choice(E, k, replace=False, p=p) for _ in range(T)],
                   dtype=np.int32).reshape(T, k)
    got = _permute_gpu(idx, E)
    ref = O.permute(idx, E)
    for a, b_, name in zip(got, ref, ("counts", "offsets", "perm", "inv_perm")):
        assert np.array_equal(a, b_), name


def test_permute_hot_expert():
    """Every token routes to expert 5 (one bucket with T rows)."""
    say("permute hot expert")
    T, k, E = 4096, 8, 64
    rng = np.random.default_rng(1)
    idx = np.stack([np.concatenate([[5], rng.choice(np.delete(np.arange(E), 5), k - 1,
                                                    replace=False)]) for _ in range(T)])
    idx = idx.astype(np.int32)
    got = _permute_gpu(idx, E)
    ref = O.permute(idx, E)
    for a, b_ in zip(got, ref):
        assert np.array_equal(a, b_)


# ------------------------------------------------------------ expert FFN

def _ffn_case(cfg, T, regime, layer=0, fmt=M.MOE_FMT_SYM):
    lay = make_layer(cfg, layer, shared=False, fmt=fmt)
    x = MI.gen_x(cfg, T)
    b = lay.buffers(T, regime)
    say("ffn %s T=%d regime=%d" % (cfg.name, T, b.regime))
    xd = f16(x)
    lay.route_permute(xd, b)
    lay.experts(xd, b)
    torch.cuda.synchronize()
    bias = MI.zipf_bias(cfg, layer)
    oi, ow, _ = O.route(x, MI.gen_router(cfg, layer), bias, cfg.k)
    assert np.array_equal(_np(b.topk_idx), oi)
    counts, offsets, perm, inv = O.permute(oi, cfg.E)
    assert np.array_equal(_np(b.offsets), offsets) and np.array_equal(_np(b.perm), perm[:T * cfg.k])
    rows = np.arange(T * cfg.k, dtype=np.int32)   # every row, every bucket edge
    used = np.unique(oi)
    blobs = OracleBlobs(cfg, layer, fmt).get(used)
    y_ref = O.expert_ffn(x, perm, offsets, blobs, cfg.H, cfg.I, cfg.E, cfg.k, cfg.g, rows=rows,
                         fmt=fmt)
    y = y_plain(b).astype(np.float64)
    # decode partials are in token order: sorted row p sits at row perm[p]
    yr = perm[rows] if b.regime & M.MOE_Y_TOKEN_ORDER else rows
    y_rows = y.sum(axis=0)[yr] if b.y_dtype != M.MOE_DTYPE_F16 else y[0][yr]
    return check_close(y_rows, y_ref, "y %s T=%d" % (cfg.name, T))


@pytest.mark.parametrize("cfg,T", [(MI.OLMOE_DECODE, 1), (MI.OLMOE_DECODE, 3), (MI.TINY, 16),
                                   (MI.E512, 4)], ids=lambda v: getattr(v, "name", str(v)))
def test_decode_token_order_y(cfg, T):
    """Decode partials written in token order (MOE_Y_TOKEN_ORDER) are the
    sorted-order partials moved to row perm[p], bit for bit, and the combine
    reading them without inv_perm gives the same output bits as the sorted
    partials combined through inv_perm."""
    say("decode token order %s T=%d" % (cfg.name, T))
    lay = make_layer(cfg, 0, shared=False)
    xd = f16(MI.gen_x(cfg, T))
    b = lay.buffers(T, M.MOE_REGIME_DECODE, partial_order=False)
    assert b.regime == M.MOE_REGIME_DECODE | M.MOE_Y_TOKEN_ORDER
    lay.route_permute(xd, b)
    lay.experts(xd, b)
    out_tok = lay.combine(b).clone()
    y_tok = b.y.clone()
    b.y.fill_(7.0)
    M.moe_expert_ffn_w4a16(xd, b.perm, b.offsets, lay.table, T, cfg.H, cfg.I, cfg.E, cfg.k,
                           cfg.g, M.MOE_REGIME_DECODE, b.y, b.y_dtype, b.y_slices)
    out_sorted = torch.empty_like(out_tok)
    M.moe_combine(b.y, b.y_dtype, b.y_slices, b.inv_perm, b.topk_w, None, None, T, cfg.H, cfg.k,
                  out_sorted)
    torch.cuda.synchronize()
    perm = _np(b.perm)
    assert np.array_equal(_np(y_tok)[:, perm, :].view(np.int32), _np(b.y).view(np.int32))
    assert np.array_equal(_np(out_tok).view(np.int16), _np(out_sorted).view(np.int16))


@pytest.mark.parametrize("cfg,T", [(MI.OLMOE_DECODE, 1), (MI.OLMOE_DECODE, 4), (MI.TINY, 2),
                                   (MI.QWEN, 1), (MI.E512, 3)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_decode_partial_order_y(cfg, T):
    """Decode partials with MOE_Y_PARTIAL_ORDER (dtype MOE_DTYPE_F32_PM) are
    the plain partials with every column moved to its partial-major position
    (the header's rule, rendered independently in pm_positions), bit for bit,
    and the combine of either layout gives the same output bits (the gated
    combine of the 60-expert layer included)."""
    say("decode partial order %s T=%d" % (cfg.name, T))
    lay = make_layer(cfg, 0)
    xd = f16(MI.gen_x(cfg, T, step=5))
    bp = lay.buffers(T, M.MOE_REGIME_DECODE, partial_order=False)
    bm = lay.buffers(T, M.MOE_REGIME_DECODE)
    assert bp.y_dtype == M.MOE_DTYPE_F32
    assert bm.y_dtype == M.MOE_DTYPE_F32_PM and bm.regime & M.MOE_Y_PARTIAL_ORDER
    outs = []
    for b in (bp, bm):
        lay.route_permute(xd, b)
        lay.experts(xd, b)
        outs.append(lay.combine(b, residual=xd, x=xd).clone())
    torch.cuda.synchronize()
    pos = pm_positions(cfg.H)
    assert np.array_equal(np.sort(pos), np.arange(cfg.H))
    assert np.array_equal(_np(bm.y)[..., pos].view(np.int32), _np(bp.y).view(np.int32))
    assert np.array_equal(_np(outs[0]).view(np.int16), _np(outs[1]).view(np.int16))


@pytest.mark.parametrize("cfg,T,regime", [
    (MI.TINY, 16, M.MOE_REGIME_DECODE), (MI.TINY, 16, M.MOE_REGIME_BATCHED),
    (MI.TINY, 1, M.MOE_REGIME_AUTO), (MI.TINY, 300, M.MOE_REGIME_BATCHED),
    (MI.OLMOE_DECODE, 1, M.MOE_REGIME_AUTO), (MI.OLMOE_DECODE, 3, M.MOE_REGIME_AUTO),
    (MI.OLMOE_DECODE, 64, M.MOE_REGIME_BATCHED), (MI.OLMOE_DECODE, 512, M.MOE_REGIME_BATCHED),
    (MI.OLMOE_DECODE, 4096, M.MOE_REGIME_BATCHED), (MI.E512, 1, M.MOE_REGIME_AUTO),
    (MI.E512, 256, M.MOE_REGIME_BATCHED), (MI.E512, 4096, M.MOE_REGIME_BATCHED),
    (G32, 3, M.MOE_REGIME_DECODE), (G32, 300, M.MOE_REGIME_BATCHED),
    (G32, 8192, M.MOE_REGIME_BATCHED),
    # small-batch kernel: K split over 1..8 waves (set by the active-expert
    # estimate), ragged T, T = 32 (the largest), group sizes 32 and 128
    (MI.TINY, 2, M.MOE_REGIME_SMALL), (MI.TINY, 16, M.MOE_REGIME_SMALL),
    (MI.TINY, 32, M.MOE_REGIME_SMALL), (MI.OLMOE_DECODE, 2, M.MOE_REGIME_SMALL),
    (MI.OLMOE_DECODE, 8, M.MOE_REGIME_AUTO), (MI.OLMOE_DECODE, 17, M.MOE_REGIME_SMALL),
    (MI.OLMOE_DECODE, 32, M.MOE_REGIME_SMALL), (MI.E512, 5, M.MOE_REGIME_SMALL),
    (MI.E512, 32, M.MOE_REGIME_SMALL), (G32, 3, M.MOE_REGIME_SMALL),
    (G32, 32, M.MOE_REGIME_SMALL)],
    ids=lambda v: getattr(v, "name", str(v)))
def test_expert_ffn(cfg, T, regime):
    _ffn_case(cfg, T, regime)


# -------------------------------------------------------- shared expert

@pytest.mark.parametrize("T", [1, 3, 8, 17, 32, 33, 100, 256, 1024, 1025, 4096])
def test_shared_ffn(T):
    cfg = MI.E512
    say("shared T=%d" % T)
    wg, wu, wd = MI.gen_shared(cfg)
    x = MI.gen_x(cfg, T)
    out = torch.empty((T, cfg.H), dtype=torch.float32, device=DEV)
    wsb = M.moe_shared_ffn_workspace_bytes(T, cfg.H, cfg.Is)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    M.moe_shared_ffn_f16(f16(x), f16(wg), f16(wu), f16(wd), T, cfg.H, cfg.Is, out, ws, wsb)
    torch.cuda.synchronize()
    toks = np.arange(T) if T <= 32 else np.sort(
        np.random.default_rng(T).choice(T, 24, replace=False))
    ref = O.shared_ffn(x, wg, wu, wd, toks=toks)
    check_close(_np(out)[toks], ref, "shared T=%d" % T)


@pytest.mark.parametrize("T", [2048, 4000, 4096, 8192])
def test_shared_ffn_wide_tiles(T):
    """The 60-expert layer's shared expert (I_s = 5632) at large batches: the
    eight-wave 256 x 256 / 128 x 256 tiles of the FP16 GEMM, with a ragged
    last row tile at 4000 tokens; 24 sampled tokens against the oracle."""
    cfg = MI.QWEN
    say("shared wide T=%d" % T)
    wg, wu, wd = MI.gen_shared(cfg)
    x = MI.gen_x(cfg, T)
    out = torch.empty((T, cfg.H), dtype=torch.float32, device=DEV)
    wsb = M.moe_shared_ffn_workspace_bytes(T, cfg.H, cfg.Is)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    M.moe_shared_ffn_f16(f16(x), f16(wg), f16(wu), f16(wd), T, cfg.H, cfg.Is, out, ws, wsb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(T)
    toks = np.sort(np.concatenate([[0, T - 1], rng.choice(np.arange(1, T - 1), 22, replace=False)]))
    ref = O.shared_ffn(x, wg, wu, wd, toks=toks)
    check_close(_np(out)[toks], ref, "shared wide T=%d" % T)


# --------------------------------------------------------------- combine

def _assert_combine_close(got, ref16, ref64, absum, nterms, extra=0.0):
    """The GPU sums n terms in fp32, the oracle in fp64: they differ by at most
    the recursive-summation bound gamma_n * sum|terms| (Higham), and each is
    then rounded once to fp16, adding at most one fp16 ulp between them.
    `extra` adds a known bound on the terms' own error (the fp32 gate)."""
    u = 2.0 ** -24
    bound = nterms * u / (1 - nterms * u) * absum + extra
    ulp = np.spacing(np.abs(ref16)).astype(np.float64)
    err = np.abs(got - ref16.astype(np.float64))
    r = err / (ulp + bound)
    i = np.unravel_index(np.argmax(r), r.shape)
    assert r[i] <= 1.0, "worst at %s: got %r ref16 %r ref64 %r (ulp %g, bound %g)" % (
        i, got[i], float(ref16[i]), ref64[i], ulp[i], bound[i])


@pytest.mark.parametrize("S,dt,shared,res", [(32, M.MOE_DTYPE_F32, False, True),
                                             (16, M.MOE_DTYPE_F32, True, False),
                                             (1, M.MOE_DTYPE_F16, True, True),
                                             (1, M.MOE_DTYPE_F32, False, False)])
def test_combine(S, dt, shared, res):
    say("combine S=%d dt=%d" % (S, dt))
    rng = np.random.default_rng(S + dt)
    T, k, H = 37, 8, 512
    ys = (rng.standard_normal((S, T * k, H)) * (0.05 if S > 1 else 0.3)).astype(
        np.float32 if dt == M.MOE_DTYPE_F32 else np.float16)
    inv = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    sh = rng.standard_normal((T, H)).astype(np.float32) if shared else None
    r = rng.standard_normal((T, H)).astype(np.float16) if res else None
    out = torch.empty((T, H), dtype=torch.float16, device=DEV)
    M.moe_combine(torch.from_numpy(ys).to(DEV), dt, S, torch.from_numpy(inv).to(DEV),
                  torch.from_numpy(w).to(DEV), None if sh is None else torch.from_numpy(sh).to(DEV),
                  None if r is None else f16(r), T, H, k, out)
    torch.cuda.synchronize()
    yo = ys.astype(np.float64).sum(axis=0)
    ref, ref64 = O.combine(yo, inv, w, None if sh is None else sh.astype(np.float64), r)
    got = _np(out).astype(np.float64)
    yabs = np.abs(ys.astype(np.float64)).sum(axis=0)
    absum = sum(w[:, j:j + 1].astype(np.float64) * yabs[inv[np.arange(T) * k + j]]
                for j in range(k))
    if sh is not None:
        absum = absum + np.abs(sh)
    if r is not None:
        absum = absum + np.abs(r.astype(np.float64))
    _assert_combine_close(got, ref, ref64, absum, S * k + 2)


def test_combine_in_place_residual():
    say("combine in place")
    rng = np.random.default_rng(3)
    T, k, H = 5, 2, 256
    ys = rng.standard_normal((1, T * k, H)).astype(np.float16)
    inv = np.arange(T * k, dtype=np.int32)
    w = np.full((T, k), 0.5, np.float32)
    r = rng.standard_normal((T, H)).astype(np.float16)
    buf = f16(r)
    M.moe_combine(torch.from_numpy(ys).to(DEV), M.MOE_DTYPE_F16, 1,
                  torch.from_numpy(inv).to(DEV), torch.from_numpy(w).to(DEV), None, buf, T, H, k,
                  buf)
    torch.cuda.synchronize()
    ref, ref64 = O.combine(ys[0].astype(np.float64), inv, w, None, r)
    absum = np.abs(r.astype(np.float64)) + 0.5 * np.abs(ys[0].astype(np.float64)).reshape(
        T, k, H).sum(axis=1)
    _assert_combine_close(_np(buf).astype(np.float64), ref, ref64, absum, k + 1)


@pytest.mark.parametrize("S,dt,T,H,res", [(44, M.MOE_DTYPE_F32, 1, 2048, True),
                                           (44, M.MOE_DTYPE_F32, 3, 2048, False),
                                           (1, M.MOE_DTYPE_F16, 37, 2048, True),
                                           (1, M.MOE_DTYPE_F16, 300, 256, False),
                                           (1, M.MOE_DTYPE_F32, 5, 1024, True)])
def test_combine_gated(S, dt, T, H, res):
    """Shared term scaled by sigmoid(x . wsg): against the oracle's fp64 gate."""
    say("combine gated S=%d dt=%d T=%d H=%d" % (S, dt, T, H))
    rng = np.random.default_rng(7 * S + T)
    k = 4
    ys = (rng.standard_normal((S, T * k, H)) * (0.05 if S > 1 else 0.3)).astype(
        np.float32 if dt == M.MOE_DTYPE_F32 else np.float16)
    inv = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    sh = rng.standard_normal((T, H)).astype(np.float32)
    r = rng.standard_normal((T, H)).astype(np.float16) if res else None
    x = rng.standard_normal((T, H)).astype(np.float16)
    wsg = (rng.standard_normal(H) * 0.02).astype(np.float16)
    out = torch.empty((T, H), dtype=torch.float16, device=DEV)
    M.moe_combine_gated(torch.from_numpy(ys).to(DEV), dt, S, torch.from_numpy(inv).to(DEV),
                        torch.from_numpy(w).to(DEV), torch.from_numpy(sh).to(DEV), f16(x),
                        f16(wsg), None if r is None else f16(r), T, H, k, out)
    torch.cuda.synchronize()
    gt = O.shared_gate(x, wsg)
    yo = ys.astype(np.float64).sum(axis=0)
    ref, ref64 = O.combine(yo, inv, w, sh.astype(np.float64), r, shared_gate=gt)
    yabs = np.abs(ys.astype(np.float64)).sum(axis=0)
    absum = sum(w[:, j:j + 1].astype(np.float64) * yabs[inv[np.arange(T) * k + j]]
                for j in range(k)) + gt[:, None] * np.abs(sh)
    if r is not None:
        absum = absum + np.abs(r.astype(np.float64))
    # the GPU's fp32 gate: its logit is within gamma_H * sum|x w| of the exact
    # one, the sigmoid's slope is at most 1/4, plus a few ulps for exp and the
    # division
    u = 2.0 ** -24
    dlogit = H * u / (1 - H * u) * (np.abs(x.astype(np.float64)) @ np.abs(wsg.astype(np.float64)))
    extra = (0.25 * dlogit + 8 * u)[:, None] * np.abs(sh)
    _assert_combine_close(_np(out).astype(np.float64), ref, ref64, absum, S * k + 2, extra)


def test_combine_gated_rejects_bad_args():
    T, k, H = 2, 4, 256
    z = torch.zeros((T * k, H), dtype=torch.float16, device=DEV)
    inv = torch.arange(T * k, dtype=torch.int32, device=DEV)
    w = torch.zeros((T, k), dtype=torch.float32, device=DEV)
    sh = torch.zeros((T, H), dtype=torch.float32, device=DEV)
    x = torch.zeros((T, H + 8), dtype=torch.float16, device=DEV)
    g = torch.zeros(H + 8, dtype=torch.float16, device=DEV)
    out = torch.empty((T, H), dtype=torch.float16, device=DEV)
    with pytest.raises(M.MoEError):
        M.moe_combine_gated(z, M.MOE_DTYPE_F16, 1, inv, w, None, x, g, None, T, H, k, out)
    with pytest.raises(M.MoEError):      # gate vector not 16-byte aligned
        M.moe_combine_gated(z, M.MOE_DTYPE_F16, 1, inv, w, sh, x, g[1:], None, T, H, k, out)


# ---------------------------------------------------------- whole layer

def _oracle_tokens(cfg, x, toks, layer=0, residual=None, shared=True):
    """Oracle layer output for selected tokens (routing, FFN, combine)."""
    xs = x[toks]
    wr = MI.gen_router(cfg, layer)
    bias = MI.zipf_bias(cfg, layer)
    idx, _, _ = O.route(xs, wr, bias, cfg.k)
    blobs = OracleBlobs(cfg, layer).get(np.unique(idx))
    sh = MI.gen_shared(cfg) if (shared and cfg.Is) else None
    gate = MI.gen_shared_gate(cfg) if (sh is not None and cfg.shared_gate) else None
    res = None if residual is None else residual[toks]
    return O.moe_layer(xs, wr, blobs, cfg.H, cfg.I, cfg.E, cfg.k, cfg.g, bias=bias,
                       shared=sh, residual=res, shared_gate_w=gate)


@pytest.mark.parametrize("cfg,T", [(MI.TINY, 16), (MI.OLMOE_DECODE, 1), (MI.OLMOE_DECODE, 8),
                                   (MI.E512, 16), (MI.OLMOE_DECODE, 64),
                                   (MI.OLMOE_DECODE, 512), (MI.OLMOE_DECODE, 4096),
                                   (MI.E512, 1), (MI.E512, 256), (MI.E512, 4096), (G32, 300),
                                   (MI.QWEN, 1), (MI.QWEN, 3), (MI.QWEN, 16), (MI.QWEN, 256),
                                   (MI.QWEN, 4096)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_layer_end_to_end(cfg, T):
    lay = make_layer(cfg, 0)
    x = MI.gen_x(cfg, T)
    res = MI.gen_residual(cfg, T) if cfg.residual else None
    b = lay.buffers(T)
    say("layer %s T=%d regime=%d" % (cfg.name, T, b.regime))
    out = lay.forward(f16(x), b, None if res is None else f16(res))
    torch.cuda.synchronize()
    if T <= 512:
        toks = np.arange(T)
    else:
        # tokens owning the first and last row of every expert bucket, plus
        # random ones
        bias = MI.zipf_bias(cfg, 0)
        oi, _, _ = O.route(x, MI.gen_router(cfg, 0), bias, cfg.k)
        _, offsets, perm, _ = O.permute(oi, cfg.E)
        rows = sample_rows(offsets, max_extra=128, seed=T)
        toks = np.unique(perm[rows] // cfg.k)
    ref = _oracle_tokens(cfg, x, toks, residual=res)
    assert np.array_equal(_np(b.topk_idx)[toks], ref["idx"])
    check_close(_np(out)[toks].astype(np.float64), ref["out_f64"], "out %s T=%d" % (cfg.name, T))
    # determinism: a second run gives the same bits
    out2 = lay.forward(f16(x), lay.buffers(T), None if res is None else f16(res))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_single_expert_top1_hot_path():
    """E = 1, k = 1 with a ragged T: one bucket of T rows, weight exactly 1."""
    cfg = MI.MoEConfig(90, "e1k1", H=256, E=1, k=1, I=128, g=64)
    lay = make_layer(cfg, 0, shared=False)
    for T, regime in [(1, M.MOE_REGIME_DECODE), (300, M.MOE_REGIME_BATCHED),
                      (5, M.MOE_REGIME_DECODE), (7, M.MOE_REGIME_SMALL),
                      (32, M.MOE_REGIME_SMALL)]:
        say("e1k1 T=%d" % T)
        x = MI.gen_x(cfg, T)
        b = lay.buffers(T, regime)
        out = lay.forward(f16(x), b)
        torch.cuda.synchronize()
        assert np.all(_np(b.topk_w) == 1.0)
        ref = _oracle_tokens(cfg, x, np.arange(T), shared=False)
        check_close(_np(out).astype(np.float64), ref["out_f64"], "e1k1 T=%d" % T)


def test_hot_expert_many_tiles():
    """A large bias sends every token to expert 5: one bucket of 4096 rows."""
    cfg = MI.OLMOE_DECODE
    lay = make_layer(cfg, 0, shared=False)
    bias = np.zeros(cfg.E, np.float32)
    bias[5] = 100.0
    lay.bias = torch.from_numpy(bias).to(DEV)
    T = 4096
    x = MI.gen_x(cfg, T)
    b = lay.buffers(T)
    say("hot expert T=%d" % T)
    xd = f16(x)
    lay.route_permute(xd, b)
    lay.experts(xd, b)
    torch.cuda.synchronize()
    oi, _, _ = O.route(x, MI.gen_router(cfg), bias, cfg.k)
    assert np.array_equal(_np(b.topk_idx), oi)
    counts, offsets, perm, _ = O.permute(oi, cfg.E)
    assert counts[5] == T
    rows = np.array([offsets[5], offsets[5] + 127, offsets[5] + 128, offsets[5] + 2049,
                     offsets[6] - 1], np.int32)
    y_ref = O.expert_ffn(x, perm, offsets, OracleBlobs(cfg, 0).get([5]), cfg.H, cfg.I, cfg.E,
                         cfg.k, cfg.g, rows=rows)
    check_close(_np(b.y)[0][rows].astype(np.float64), y_ref, "hot expert y")


def test_hot_expert_small_batch():
    """Every one of 32 tokens routes to expert 5: the small-batch kernel's
    largest row count (32, one MFMA column operand) next to experts with one
    or two rows."""
    cfg = MI.OLMOE_DECODE
    lay = make_layer(cfg, 0, shared=False)
    bias = np.zeros(cfg.E, np.float32)
    bias[5] = 100.0
    lay.bias = torch.from_numpy(bias).to(DEV)
    T = 32
    x = MI.gen_x(cfg, T)
    b = lay.buffers(T, M.MOE_REGIME_SMALL)
    say("hot expert small T=%d" % T)
    xd = f16(x)
    lay.route_permute(xd, b)
    lay.experts(xd, b)
    torch.cuda.synchronize()
    oi, _, _ = O.route(x, MI.gen_router(cfg), bias, cfg.k)
    assert np.array_equal(_np(b.topk_idx), oi)
    counts, offsets, perm, _ = O.permute(oi, cfg.E)
    assert counts[5] == T
    rows = np.arange(T * cfg.k, dtype=np.int32)
    y_ref = O.expert_ffn(x, perm, offsets, OracleBlobs(cfg, 0).get(np.unique(oi)), cfg.H, cfg.I,
                         cfg.E, cfg.k, cfg.g, rows=rows)
    check_close(_np(b.y)[0][rows].astype(np.float64), y_ref, "hot expert small y")


def test_small_batch_idle_waves_and_parts():
    """Small-batch kernel with 14 fused blocks dealt four to a workgroup (the
    last workgroup has two idle waves), the rows staged in two parts of K
    (32 rows of H = 1024), and 32 rows on each of the 16 routed experts."""
    cfg = MI.MoEConfig(92, "h1024_i448_e160", H=1024, E=160, k=16, I=448, g=64)
    lay = make_layer(cfg, 0, shared=False)
    bias = np.zeros(cfg.E, np.float32)
    bias[:cfg.k] = 100.0
    lay.bias = torch.from_numpy(bias).to(DEV)
    T = 32
    x = MI.gen_x(cfg, T)
    b = lay.buffers(T, M.MOE_REGIME_SMALL)
    say("small batch idle waves T=%d" % T)
    xd = f16(x)
    lay.route_permute(xd, b)
    lay.experts(xd, b)
    torch.cuda.synchronize()
    oi, _, _ = O.route(x, MI.gen_router(cfg), bias, cfg.k)
    assert np.array_equal(_np(b.topk_idx), oi)
    counts, offsets, perm, _ = O.permute(oi, cfg.E)
    assert np.all(counts[:cfg.k] == T)
    rows = np.arange(T * cfg.k, dtype=np.int32)
    y_ref = O.expert_ffn(x, perm, offsets, OracleBlobs(cfg, 0).get(range(cfg.k)), cfg.H, cfg.I,
                         cfg.E, cfg.k, cfg.g, rows=rows)
    check_close(_np(b.y)[0][rows].astype(np.float64), y_ref, "small batch idle waves y")


@pytest.mark.parametrize("H,I,g,E,k,T", [(1024, 448, 64, 160, 16, 1), (1024, 448, 64, 160, 16, 4),
                                          (2048, 256, 32, 16, 4, 2), (2048, 256, 64, 16, 4, 3),
                                          (512, 192, 32, 16, 4, 4)])
def test_decode_row_groups_and_shapes(H, I, g, E, k, T):
    """Decode regime at the instantiated H and group sizes with every token
    routed to the same k experts, so each expert holds T rows: one group of
    1..4 rows sharing each weight unpack (down chunks unpacked ahead for up
    to two rows, where used above), partials written in token order."""
    cfg = MI.MoEConfig(93, "dec_h%d_g%d_t%d" % (H, g, T), H=H, E=E, k=k, I=I, g=g)
    say("decode groups %s" % cfg.name)
    lay = make_layer(cfg, 0, shared=False)
    bias = np.zeros(cfg.E, np.float32)
    bias[3:3 + cfg.k] = 100.0
    lay.bias = torch.from_numpy(bias).to(DEV)
    x = MI.gen_x(cfg, T)
    b = lay.buffers(T, M.MOE_REGIME_DECODE)
    assert b.regime & ~M.MOE_Y_PARTIAL_ORDER == M.MOE_REGIME_DECODE | M.MOE_Y_TOKEN_ORDER
    xd = f16(x)
    lay.route_permute(xd, b)
    lay.experts(xd, b)
    out = lay.combine(b)
    torch.cuda.synchronize()
    oi, ow, _ = O.route(x, MI.gen_router(cfg), bias, cfg.k)
    assert np.array_equal(_np(b.topk_idx), oi)
    counts, offsets, perm, inv = O.permute(oi, cfg.E)
    assert np.all(counts[3:3 + cfg.k] == T)
    rows = np.arange(T * cfg.k, dtype=np.int32)
    blobs = OracleBlobs(cfg, 0).get(range(3, 3 + cfg.k))
    y_ref = O.expert_ffn(x, perm, offsets, blobs, cfg.H, cfg.I, cfg.E, cfg.k, cfg.g, rows=rows)
    check_close(y_plain(b).astype(np.float64).sum(axis=0)[perm[rows]], y_ref, "y %s" % cfg.name)
    ref = O.moe_layer(x, MI.gen_router(cfg), blobs, cfg.H, cfg.I, cfg.E, cfg.k, cfg.g,
                      bias=bias)   # only the routed experts' blobs are packed
    check_close(_np(out).astype(np.float64), ref["out_f64"], "out %s" % cfg.name)


def test_zero_tokens_is_noop():
    cfg = MI.OLMOE_DECODE
    lay = make_layer(cfg, 0, shared=False)
    b = lay.buffers(0)
    lay.forward(f16(np.zeros((0, cfg.H), np.float16)), b)
    torch.cuda.synchronize()
    assert np.all(_np(b.offsets) == 0) and np.all(_np(b.counts) == 0)


@pytest.mark.parametrize("cfg,T", [(MI.E512, 1), (MI.QWEN, 8)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_layer_shared_overlap_matches_serial_and_graph(cfg, T):
    """The shared expert on a side stream (forked at the layer's start, joined
    before the combine) gives the same bits as the one-stream order, eagerly
    and in a captured graph replayed several times with eager work between."""
    say("shared overlap %s T=%d" % (cfg.name, T))
    lay = make_layer(cfg, 0)
    x = f16(MI.gen_x(cfg, T))
    ref = lay.forward(x, lay.buffers(T), overlap_shared=False).clone()
    b = lay.buffers(T)
    out = lay.forward(x, b, overlap_shared=True).clone()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    bg = lay.buffers(T)
    lay.forward(x, bg, overlap_shared=True)   # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        og = lay.forward(x, bg, overlap_shared=True)
    for _ in range(3):
        og.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(og.view(torch.int16), ref.view(torch.int16))
        lay.forward(x, b, overlap_shared=True)   # eager work between replays
        torch.cuda.synchronize()


# ------------------------------------------------------ workspace recovery

def test_workspace_clear_recovers_a_stale_ticket():
    """A fused route+permute workspace whose ticket was left non-zero (as by
    an interrupted call) skips the top-k; moe_workspace_clear restores it.
    The fill touches exactly the bytes asked for, at any alignment."""
    cfg = MI.OLMOE_DECODE
    T = 1
    say("workspace clear")
    x = MI.gen_x(cfg, T, step=3)
    wr = MI.gen_router(cfg)
    n = T * cfg.k
    wsb = M.moe_route_permute_workspace_bytes(T, cfg.k, cfg.E)
    ws = torch.zeros(wsb + 64, dtype=torch.uint8, device=DEV)
    # a stale ticket far from any arrival count: no workgroup takes the last
    # ticket, so no top-k runs and the outputs keep their fill
    ws[:4] = torch.tensor([0xE8, 0x03, 0, 0], dtype=torch.uint8)   # 1000
    outs = [torch.full((T, cfg.k), -7, dtype=torch.int32, device=DEV),
            torch.empty((T, cfg.k), dtype=torch.float32, device=DEV),
            torch.empty(cfg.E, dtype=torch.int32, device=DEV),
            torch.empty(cfg.E + 1, dtype=torch.int32, device=DEV),
            torch.empty(n, dtype=torch.int32, device=DEV),
            torch.empty(n, dtype=torch.int32, device=DEV)]
    M.moe_route_permute(f16(x), f16(wr), None, T, cfg.H, cfg.E, cfg.k, 0, *outs, ws, wsb)
    torch.cuda.synchronize()
    assert np.all(_np(outs[0]) == -7)        # the stale ticket made every workgroup skip
    M.moe_workspace_clear(ws, wsb)
    outs[0].fill_(-7)
    M.moe_route_permute(f16(x), f16(wr), None, T, cfg.H, cfg.E, cfg.k, 0, *outs, ws, wsb)
    torch.cuda.synchronize()
    oi, _, _ = O.route(x, wr, None, cfg.k)
    assert np.array_equal(_np(outs[0]), oi)
    assert int(ws[:4].view(torch.int32).item()) == 0
    # exact extent at odd addresses and sizes
    buf = torch.full((4096,), 0xAB, dtype=torch.uint8, device=DEV)
    for off, nb in [(3, 1), (5, 100), (16, 2048), (7, 3001), (0, 4096)]:
        buf.fill_(0xAB)
        M.moe_workspace_clear(buf.data_ptr() + off, nb)
        torch.cuda.synchronize()
        v = _np(buf)
        assert np.all(v[off:off + nb] == 0) and np.all(v[:off] == 0xAB) and \
            np.all(v[off + nb:] == 0xAB), (off, nb)


# ------------------------------------------------------ zero-point format

@pytest.mark.parametrize("cfg", [MI.TINY, MI.OLMOE_DECODE, MI.E512, G32], ids=lambda c: c.name)
def test_quantize_zero_point_bit_exact(cfg):
    """The library's zero-point quantiser makes the oracle's decisions: the
    canonical blobs (codes, scales, zero points) are identical bytes."""
    say("quantize zp %s" % cfg.name)
    ex = [0, 1, cfg.E - 1]
    _, canon = device_experts(cfg, 0, experts=ex, fmt=M.MOE_FMT_ZP)
    ob = OracleBlobs(cfg, 0, O.FMT_ZP).get(ex)
    assert M.moe_blob_layout_fmt(cfg.H, cfg.I, cfg.g, M.MOE_FMT_ZP) == \
        tuple(O.blob_layout(cfg.H, cfg.I, cfg.g, O.FMT_ZP))
    for e in ex:
        assert np.array_equal(_np(canon[e]), ob[e]), "expert %d blob differs" % e


@pytest.mark.parametrize("cfg", [MI.TINY, G32], ids=lambda c: c.name)
def test_prepack_zero_point_layout_and_round_trip(cfg):
    say("prepack zp %s" % cfg.name)
    dev, canon = device_experts(cfg, 0, experts=[0, 3], fmt=M.MOE_FMT_ZP)
    for e in (0, 3):
        ref = _numpy_prepack(_np(canon[e]), cfg.H, cfg.I, cfg.g, O.FMT_ZP)
        assert np.array_equal(_np(dev[e]), ref)
    back = torch.empty_like(dev)
    M.moe_unpack_experts_fmt(dev, cfg.E, cfg.H, cfg.I, cfg.g, M.MOE_FMT_ZP, back)
    torch.cuda.synchronize()
    for e in (0, 3):
        assert np.array_equal(_np(back[e]), _np(canon[e]))


@pytest.mark.parametrize("cfg,T,regime", [
    (MI.TINY, 16, M.MOE_REGIME_DECODE), (MI.TINY, 16, M.MOE_REGIME_SMALL),
    (MI.TINY, 16, M.MOE_REGIME_BATCHED), (MI.TINY, 300, M.MOE_REGIME_BATCHED),
    (MI.OLMOE_DECODE, 1, M.MOE_REGIME_AUTO), (MI.OLMOE_DECODE, 3, M.MOE_REGIME_AUTO),
    (MI.OLMOE_DECODE, 8, M.MOE_REGIME_AUTO), (MI.OLMOE_DECODE, 32, M.MOE_REGIME_SMALL),
    (MI.OLMOE_DECODE, 64, M.MOE_REGIME_BATCHED), (MI.OLMOE_DECODE, 512, M.MOE_REGIME_BATCHED),
    (MI.OLMOE_DECODE, 4096, M.MOE_REGIME_BATCHED), (MI.E512, 1, M.MOE_REGIME_AUTO),
    (MI.E512, 256, M.MOE_REGIME_BATCHED), (G32, 3, M.MOE_REGIME_DECODE),
    (G32, 32, M.MOE_REGIME_SMALL), (G32, 300, M.MOE_REGIME_BATCHED)],
    ids=lambda v: getattr(v, "name", str(v)))
def test_expert_ffn_zero_point(cfg, T, regime):
    """Routed FFN from zero-point blobs in every regime, every row against the
    oracle's zero-point decoder."""
    _ffn_case(cfg, T, regime, fmt=M.MOE_FMT_ZP)


@pytest.mark.parametrize("cfg,T", [(MI.OLMOE_DECODE, 1), (MI.OLMOE_DECODE, 16),
                                   (MI.E512, 300)], ids=lambda v: getattr(v, "name", str(v)))
def test_layer_zero_point(cfg, T):
    """Whole layers (route, permute, zero-point FFN, shared expert, combine)."""
    lay = make_layer(cfg, 0, fmt=M.MOE_FMT_ZP)
    x = MI.gen_x(cfg, T, step=5)
    res = MI.gen_residual(cfg, T) if cfg.residual else None
    b = lay.buffers(T)
    assert b.regime & M.MOE_W4_ZERO_POINT
    say("layer zp %s T=%d regime=%d" % (cfg.name, T, b.regime))
    out = lay.forward(f16(x), b, None if res is None else f16(res))
    torch.cuda.synchronize()
    wr = MI.gen_router(cfg, 0)
    bias = MI.zipf_bias(cfg, 0)
    idx, _, _ = O.route(x, wr, bias, cfg.k)
    sh = MI.gen_shared(cfg) if cfg.Is else None
    ref = O.moe_layer(x, wr, OracleBlobs(cfg, 0, O.FMT_ZP).get(np.unique(idx)), cfg.H, cfg.I,
                      cfg.E, cfg.k, cfg.g, bias=bias, shared=sh, residual=res, fmt=O.FMT_ZP)
    assert np.array_equal(_np(b.topk_idx), ref["idx"])
    check_close(_np(out).astype(np.float64), ref["out_f64"], "zp layer %s T=%d" % (cfg.name, T))


E33 = MI.MoEConfig(89, "h512_e33_k16", H=512, E=33, k=16, I=128, g=64)


@pytest.mark.parametrize("cfg", [MI.TINY, MI.QWEN, E33, MI.OLMOE_DECODE, MI.E512],
                         ids=lambda c: c.name)
@pytest.mark.parametrize("case", ["plain", "renorm", "ties", "zero"])
def test_route_permute_one_token(cfg, case):
    """One token through the fused route+sort (the decode path; up to 64
    experts it selects and sorts in registers): routing, weights, counts,
    offsets, permutation against the oracle, with renormalisation, exact ties
    (duplicated router rows: lower index first) and a zero input (all logits
    equal: experts 0..k-1)."""
    say("route_permute one token %s %s" % (cfg.name, case))
    T, k, E = 1, cfg.k, cfg.E
    x = MI.gen_x(cfg, T, step=31)
    wr = MI.gen_router(cfg)
    if case == "ties":
        wr[E - 1] = wr[1]
        wr[E // 2] = wr[1]
        wr[2] = wr[0]
    if case == "zero":
        x[:] = 0.0
    b = MI.zipf_bias(cfg) if case != "zero" else None
    renorm = case == "renorm"
    outs = [torch.full((T, k), -7, dtype=torch.int32, device=DEV),
            torch.full((T, k), -7.0, dtype=torch.float32, device=DEV),
            torch.full((E,), -7, dtype=torch.int32, device=DEV),
            torch.full((E + 1,), -7, dtype=torch.int32, device=DEV),
            torch.full((k,), -7, dtype=torch.int32, device=DEV),
            torch.full((k,), -7, dtype=torch.int32, device=DEV)]
    wsb = M.moe_route_permute_workspace_bytes(T, k, E)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    for rep in range(2):
        M.moe_route_permute(f16(x), f16(wr), None if b is None else torch.from_numpy(b).to(DEV),
                            T, cfg.H, E, k, M.MOE_RENORM if renorm else 0, *outs, ws, wsb)
        torch.cuda.synchronize()
        oi, ow, _ = O.route(x, wr, b, k, renorm)
        assert np.array_equal(_np(outs[0]), oi)
        assert np.max(np.abs(_np(outs[1]) - ow)) <= WTOL
        for got, ref, name in zip(outs[2:], O.permute(oi, E), ("counts", "offsets", "perm", "inv")):
            assert np.array_equal(_np(got), ref), name
        assert int(_np(ws[:4].view(torch.int32))[0]) == 0
    if case == "zero":
        assert np.array_equal(oi[0], np.arange(k))
