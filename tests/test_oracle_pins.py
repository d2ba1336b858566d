"""Pins of the CPU oracle against facts that do not come from the oracle:
closed forms, textbook routines, brute force, exhaustive small cases and
independent implementations (numpy's fp16 codec, numpy stable sorts, dense
numpy fp64 FFNs).  A plausible slip in the oracle (dropped term, wrong sign,
transposed operand, wrong nibble, wrong tie-break) fails at least one test.
"""
import itertools
import math

import numpy as np
import pytest

import oracle as O
import moe_inputs as MI


# ------------------------------------------------------------------ fp16

def test_f16_decode_exhaustive_matches_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    ours = O.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # sign of zero is kept
    assert math.copysign(1.0, ours[0x8000]) == -1.0


def test_f16_encode_rne_matches_numpy():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 6, 200000),
        rng.uniform(-70000, 70000, 20000),
    ])
    # exact halfway points between neighbouring fp16 values (ties to even)
    allf = np.arange(0, 0x7c00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (allf[:-1] + allf[1:]) / 2
    edge = np.array([0.0, -0.0, 65504.0, 65519.999, 65520.0, 1e6, -1e6, 2.0 ** -24,
                     2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -12)])
    v = np.concatenate([v, mids, -mids, edge])
    ours = O.f64_to_f16(v)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------- quantiser

def _unpack(q):
    lo = (q & 15).astype(np.int64) - 8
    hi = (q >> 4).astype(np.int64) - 8
    out = np.empty((q.shape[0], q.shape[1] * 2), np.int64)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


@pytest.mark.parametrize("g", [32, 64, 128])
def test_quantiser_error_bound_closed_form(g):
    rng = np.random.default_rng(g)
    w = (rng.standard_normal((37, 4 * g)) * 0.02).astype(np.float32)
    w[3, :g] = 0.0                         # an all-zero group: s = 0, q = 0
    q, s = O.quantize_rows(w, g)
    codes = _unpack(q)
    assert codes.min() >= -7 and codes.max() <= 7
    deq = O.dequant_rows(q, s, g)
    sv = O.f16_to_f64(s)                          # [rows, K/g]
    amax = np.abs(w.astype(np.float64)).reshape(37, -1, g).max(axis=2)
    s_exact = amax / 7.0
    bound = sv / 2 * (1 + 1e-6) + 7 * np.abs(sv - s_exact) + 1e-30
    err = np.abs(w.astype(np.float64) - deq).reshape(37, -1, g)
    assert np.all(err <= bound[:, :, None])
    # dequantised value is exactly code * scale
    assert np.array_equal(deq, codes * np.repeat(sv, g, axis=1))
    # the element of largest magnitude maps to +-7 (fp16 rounding of s moves
    # amax/s by at most 7*2^-11 < 0.5)
    wg = w.reshape(37, -1, g)
    cg = codes.reshape(37, -1, g)
    am = np.abs(wg).argmax(axis=2)
    for r in range(37):
        for G in range(wg.shape[1]):
            if amax[r, G] == 0:
                assert np.all(cg[r, G] == 0) and sv[r, G] == 0
                continue
            assert abs(cg[r, G, am[r, G]]) == 7
            assert np.sign(cg[r, G, am[r, G]]) == np.sign(wg[r, G, am[r, G]])


def test_quantiser_exact_round_trip():
    """w = q * 2^-m with group max |q| = 7 round-trips exactly."""
    rng = np.random.default_rng(7)
    g = 64
    codes = rng.integers(-7, 8, (16, 4 * g))
    for r in range(16):
        for G in range(4):
            codes[r, G * g + rng.integers(g)] = 7 * (1 if rng.random() < 0.5 else -1)
    m = rng.integers(3, 12, (16, 4))
    w = (codes * np.repeat(2.0 ** -m.astype(np.float64), g, axis=1)).astype(np.float32)
    q, s = O.quantize_rows(w, g)
    assert np.array_equal(_unpack(q), codes)
    assert np.array_equal(O.f16_to_f64(s), 2.0 ** -m.astype(np.float64))
    assert np.array_equal(O.dequant_rows(q, s, g), w.astype(np.float64))


def test_pack_nibble_order_and_decode_all_bytes():
    # every pair of codes packs as low = even element, high = odd element
    pairs = np.array(list(itertools.product(range(-7, 8), repeat=2)))
    w = np.zeros((1, 2 * len(pairs) + 0), np.float32)
    w[0, 0::2] = pairs[:, 0]
    w[0, 1::2] = pairs[:, 1]
    # groups of 2 elements would change scales; use one scale of 1 by forcing
    # a 7 in each group of 450 (the whole row is one group)
    g = w.shape[1]
    w[0, 0] = 7.0
    pairs[0, 0] = 7
    q, s = O.quantize_rows(w, g)
    assert O.f16_to_f64(s)[0, 0] == 1.0
    expect = ((pairs[:, 1] + 8) << 4) | (pairs[:, 0] + 8)
    assert np.array_equal(q[0], expect.astype(np.uint8))
    # decoding every one of the 256 byte values (u = 0 included)
    qb = np.arange(256, dtype=np.uint8).reshape(1, 256)
    sb = np.array([[0x3c00]], np.uint16)       # scale 1.0, one group of 512
    d = O.dequant_rows(qb, sb, 512)
    assert np.array_equal(d[0, 0::2], (np.arange(256) & 15) - 8.0)
    assert np.array_equal(d[0, 1::2], (np.arange(256) >> 4) - 8.0)


@pytest.mark.parametrize("cfg,expect", [(MI.OLMOE_DECODE, 3244032), (MI.E512, 1622016),
                                        (MI.TINY, 208896)])
def test_blob_bytes_closed_form(cfg, expect):
    """bytes = P * 4 / 8 + one fp16 scale per block of g (the local-inference
    explainer's step-1 formula with per-block scale overhead)."""
    P = 3 * cfg.H * cfg.I
    closed = P * 4 // 8 + (P // cfg.g) * 2
    off, tot = O.blob_layout(cfg.H, cfg.I, cfg.g)
    assert tot == closed == expect
    assert all(o % 256 == 0 for o in off)


# ---------------------------------------------------------------- router

def _pinned_logits_numpy(x16, w16):
    """Independent float32 rendering of the pinned order (chunks of 8 to
    partial c mod 64, in order, then the xor butterfly)."""
    x = x16.astype(np.float32)
    w = w16.astype(np.float32)
    T, H = x.shape
    E = w.shape[0]
    out = np.empty((T, E), np.float32)
    for t in range(T):
        for e in range(E):
            part = np.zeros(64, np.float32)
            prod = x[t] * w[e]
            for c in range(H // 8):
                for i in range(8):
                    part[c % 64] = np.float32(part[c % 64] + prod[c * 8 + i])
            for st in (32, 16, 8, 4, 2, 1):
                part = (part + part[np.arange(64) ^ st]).astype(np.float32)
            out[t, e] = part[0]
    return out


def test_logits_within_recursive_summation_bound_and_pinned_order():
    cfg = MI.OLMOE_DECODE
    x = MI.gen_x(cfg, 3)
    wr = MI.gen_router(cfg)[:16]
    _, _, l = O.route(x, wr, None, k=2)
    exact = x.astype(np.float64) @ wr.astype(np.float64).T
    absd = np.abs(x.astype(np.float64)) @ np.abs(wr.astype(np.float64)).T
    u = 2.0 ** -24
    n = cfg.H
    gamma = n * u / (1 - n * u)
    assert np.all(np.abs(l - exact) <= gamma * absd)
    assert np.array_equal(l, _pinned_logits_numpy(x, wr))


def test_logit_bias_added_after_dot():
    cfg = MI.TINY
    x = MI.gen_x(cfg, 4)
    wr = MI.gen_router(cfg)
    b = np.linspace(-1, 1, cfg.E).astype(np.float32)
    _, _, l0 = O.route(x, wr, None, k=2)
    _, _, l1 = O.route(x, wr, b, k=2)
    assert np.array_equal(l1, (l0 + b).astype(np.float32))


def test_topk_matches_stable_argsort():
    cfg = MI.E512
    x = MI.gen_x(cfg, 8)
    wr = MI.gen_router(cfg)
    bias = MI.zipf_bias(cfg)
    idx, w, l = O.route(x, wr, bias, k=cfg.k)
    ref = np.argsort(-l, axis=1, kind="stable")[:, :cfg.k]
    assert np.array_equal(idx, ref)
    # weights decrease along the top-k order (softmax is monotone)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_topk_zero_input_lower_index_tiebreak():
    cfg = MI.OLMOE_DECODE
    x = np.zeros((2, cfg.H), np.float16)
    wr = MI.gen_router(cfg)
    idx, w, _ = O.route(x, wr, None, k=cfg.k)
    assert np.array_equal(idx, np.tile(np.arange(cfg.k), (2, 1)))
    assert np.all(w == np.float32(1.0 / cfg.E))


def test_topk_exhaustive_ties_small_E():
    """E = 5, every assignment of experts to 3 router rows (ties), all k."""
    H = 64
    rng = np.random.default_rng(3)
    base = rng.standard_normal((3, H)).astype(np.float16)
    x = rng.standard_normal((1, H)).astype(np.float16)
    for pattern in itertools.product(range(3), repeat=5):
        wr = base[list(pattern)]
        for k in range(1, 6):
            idx, w, l = O.route(x, wr, None, k=k)
            ref = np.argsort(-l[0], kind="stable")[:k]
            assert np.array_equal(idx[0], ref), (pattern, k)


def test_softmax_invariants_and_zipf_closed_form():
    cfg = MI.E512
    E = cfg.E
    x = MI.gen_x(cfg, 2)
    wr = np.zeros((E, cfg.H), np.float16)          # logits = bias exactly
    bias = MI.zipf_bias(cfg)
    idx, w, l = O.route(x, wr, bias, k=E)
    assert np.array_equal(l[0], bias)
    # Zipf closed form: p_e = rank_e^-s / H_{E,s}, ranks from the bias
    s = cfg.zipf_s
    rank = np.rint(np.exp(-bias.astype(np.float64) / s)).astype(np.int64)
    assert sorted(rank) == list(range(1, E + 1))
    HEs = sum(r ** -s for r in range(1, E + 1))
    # bias was rounded to fp32, so p is the softmax of the rounded bias:
    # relative error at most ~ E * 2^-24 * max|bias| in the exponent
    p_closed = rank.astype(np.float64) ** -s / HEs
    got = np.empty(E)
    got[idx[0]] = w[0]
    assert np.allclose(got, p_closed, rtol=2e-6, atol=0)
    assert abs(w[0].astype(np.float64).sum() - 1.0) < E * 2.0 ** -23
    # generic logits: sum over all experts is one, and renorm sums top-k to one
    wr2 = MI.gen_router(cfg)
    _, w_all, _ = O.route(x, wr2, bias, k=E)
    assert np.allclose(w_all.astype(np.float64).sum(axis=1), 1.0, atol=E * 2.0 ** -23)
    _, w_rn, _ = O.route(x, wr2, bias, k=cfg.k, renorm=True)
    assert np.allclose(w_rn.astype(np.float64).sum(axis=1), 1.0, atol=1e-6)


# ----------------------------------------------------------- permutation

@pytest.mark.parametrize("T,k,E", [(16, 2, 8), (1, 8, 64), (333, 10, 512), (7, 3, 4)])
def test_permutation_brute_force_and_invariants(T, k, E):
    rng = np.random.default_rng(T)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, inv = O.permute(idx, E)
    flat = idx.reshape(-1)
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(inv[perm], np.arange(T * k))
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(flat[seg] == e)


def test_permutation_empty():
    idx = np.zeros((0, 4), np.int32)
    counts, offsets, perm, inv = O.permute(idx, 8)
    assert counts.sum() == 0 and np.all(offsets == 0) and perm.size == 0


# ----------------------------------------------------------- expert FFN

def _silu(a):
    return a / (1 + np.exp(-a))


def _dense_swiglu(x, wg, wu, wd):
    """Textbook dense SwiGLU FFN, fp64: y = Wd (silu(Wg x) * (Wu x))."""
    return (_silu(x @ wg.T) * (x @ wu.T)) @ wd.T


def _exact_int4_weights(rng, rows, K, g):
    codes = rng.integers(-7, 8, (rows, K))
    for r in range(rows):
        for G in range(K // g):
            codes[r, G * g] = 7
    m = rng.integers(5, 9, (rows, K // g)).astype(np.float64)
    return (codes * np.repeat(2.0 ** -m, g, axis=1)).astype(np.float32)


def test_single_expert_top1_equals_dense_ffn():
    """E = 1, k = 1: the routing weight is exactly 1 and the layer is a dense
    SwiGLU FFN of the (exactly representable) INT4 weights."""
    rng = np.random.default_rng(11)
    H, I, g, T = 128, 256, 64, 5
    wg = _exact_int4_weights(rng, I, H, g)
    wu = _exact_int4_weights(rng, I, H, g)
    wd = _exact_int4_weights(rng, H, I, g)
    blob = O.pack_expert(wg, wu, wd, g)
    x = rng.standard_normal((T, H)).astype(np.float16)
    wr = rng.standard_normal((1, H)).astype(np.float16)
    r = O.moe_layer(x, wr, [blob], H, I, 1, 1, g)
    assert np.all(r["w"] == 1.0) and np.all(r["idx"] == 0)
    dense = _dense_swiglu(x.astype(np.float64), wg.astype(np.float64),
                          wu.astype(np.float64), wd.astype(np.float64))
    assert np.allclose(r["y"], dense, rtol=1e-12, atol=1e-12)
    assert np.allclose(r["out_f64"], dense, rtol=1e-12, atol=1e-12)
    # final rounding is fp16 RNE of the fp64 value
    assert np.array_equal(r["out"], r["out_f64"].astype(np.float16))


def test_generic_ffn_matches_dense_dequantised():
    cfg = MI.TINY
    T = cfg.T[0]
    x = MI.gen_x(cfg, T)
    wr = MI.gen_router(cfg)
    blobs = [O.pack_expert(*MI.gen_expert(cfg, 0, e), cfg.g) for e in range(cfg.E)]
    r = O.moe_layer(x, wr, blobs, cfg.H, cfg.I, cfg.E, cfg.k, cfg.g)
    xs = x.astype(np.float64)
    out = np.zeros((T, cfg.H))
    for t in range(T):
        for j in range(cfg.k):
            e = r["idx"][t, j]
            gq, uq, dq, gs, us, ds = O.blob_sections(blobs[e], cfg.H, cfg.I, cfg.g)
            Wg = _unpack(gq) * np.repeat(O.f16_to_f64(gs), cfg.g, axis=1)
            Wu = _unpack(uq) * np.repeat(O.f16_to_f64(us), cfg.g, axis=1)
            Wd = _unpack(dq) * np.repeat(O.f16_to_f64(ds), cfg.g, axis=1)
            yv = _dense_swiglu(xs[t:t + 1], Wg, Wu, Wd)[0]
            p = r["inv_perm"][t * cfg.k + j]
            assert np.allclose(r["y"][p], yv, rtol=1e-11, atol=1e-13)
            out[t] += float(r["w"][t, j]) * yv
    assert np.allclose(r["out_f64"], out, rtol=1e-11, atol=1e-13)


def test_all_experts_identical():
    cfg = MI.TINY
    T = 6
    x = MI.gen_x(cfg, T)
    wr = MI.gen_router(cfg)
    blob = O.pack_expert(*MI.gen_expert(cfg, 0, 0), cfg.g)
    r = O.moe_layer(x, wr, [blob] * cfg.E, cfg.H, cfg.I, cfg.E, cfg.k, cfg.g)
    one = O.moe_layer(x, wr[:1], [blob], cfg.H, cfg.I, 1, 1, cfg.g)
    wsum = r["w"].astype(np.float64).sum(axis=1, keepdims=True)
    assert np.allclose(r["out_f64"], wsum * one["y"], rtol=1e-12, atol=1e-14)


def test_zero_input_gives_residual():
    cfg = MI.TINY
    T = 4
    x = np.zeros((T, cfg.H), np.float16)
    wr = MI.gen_router(cfg)
    blobs = [O.pack_expert(*MI.gen_expert(cfg, 0, e), cfg.g) for e in range(cfg.E)]
    res = MI.gen_residual(cfg, T)
    r = O.moe_layer(x, wr, blobs, cfg.H, cfg.I, cfg.E, cfg.k, cfg.g, residual=res)
    assert np.all(r["y"] == 0.0)
    assert np.array_equal(r["out"].view(np.uint16), res.view(np.uint16))


def test_combine_one_hot_weights():
    rng = np.random.default_rng(5)
    T, k, H = 3, 4, 32
    y = rng.standard_normal((T * k, H))
    inv = rng.permutation(T * k).astype(np.int32)
    w = np.zeros((T, k), np.float32)
    hot = rng.integers(0, k, T)
    w[np.arange(T), hot] = 1.0
    out, o64 = O.combine(y, inv, w)
    for t in range(T):
        assert np.array_equal(o64[t], y[inv[t * k + hot[t]]])
        assert np.array_equal(out[t], y[inv[t * k + hot[t]]].astype(np.float16))


def test_shared_ffn_equals_dense():
    cfg = MI.E512
    wg, wu, wd = MI.gen_shared(cfg)
    x = MI.gen_x(cfg, 3)
    s = O.shared_ffn(x, wg, wu, wd)
    d = _dense_swiglu(x.astype(np.float64), wg.astype(np.float64), wu.astype(np.float64),
                      wd.astype(np.float64))
    assert np.allclose(s, d, rtol=1e-11, atol=1e-13)
    s2 = O.shared_ffn(x, wg, wu, wd, toks=[2, 0])
    assert np.array_equal(s2, s[[2, 0]])


# ------------------------------------------------- gated shared expert

def test_shared_gate_dot_matches_pinned_router_logit():
    """The gate's logit is a dot of x with one more fp16 row: the oracle's
    fp64 gate must be the sigmoid of a value within the recursive-summation
    bound of the router's separately pinned fp32 logit for that row."""
    cfg = MI.QWEN
    x = MI.gen_x(cfg, 6)
    wsg = MI.gen_shared_gate(cfg)
    gt = O.shared_gate(x, wsg)
    _, _, l = O.route(x, wsg[None, :], None, k=1)
    absd = np.abs(x.astype(np.float64)) @ np.abs(wsg.astype(np.float64))
    u = 2.0 ** -24
    gamma = cfg.H * u / (1 - cfg.H * u)
    a = np.log(gt / (1.0 - gt))          # logit recovered from the gate
    assert np.all(np.abs(a - l[:, 0].astype(np.float64)) <= gamma * absd + 1e-12)
    assert np.all((gt > 0.5) == (l[:, 0] > 0))


def test_shared_gate_special_cases():
    cfg = MI.QWEN
    x = MI.gen_x(cfg, 5)
    wsg = MI.gen_shared_gate(cfg)
    # zero gate vector: exactly one half
    assert np.all(O.shared_gate(x, np.zeros(cfg.H, np.float16)) == 0.5)
    # negating the vector mirrors the gate about one half
    g1 = O.shared_gate(x, wsg)
    g2 = O.shared_gate(x, -wsg)
    assert np.allclose(g1 + g2, 1.0, rtol=0, atol=1e-15)
    # saturation: logit +H gives exactly 1, -H exactly 0 in fp64
    ones = np.ones((2, cfg.H), np.float16)
    assert np.all(O.shared_gate(ones, np.ones(cfg.H, np.float16)) == 1.0)
    assert np.all(O.shared_gate(ones, -np.ones(cfg.H, np.float16)) == 0.0)
    # token selection
    assert np.array_equal(O.shared_gate(x, wsg, toks=[4, 1]), g1[[4, 1]])


def test_gated_combine_scales_only_the_shared_term():
    """Gating is the same as pre-scaling the shared rows; the routed and
    residual terms are untouched (gate 0 removes only the shared term, gate 1
    is the ungated combine)."""
    rng = np.random.default_rng(8)
    T, k, H = 5, 4, 64
    y = rng.standard_normal((T * k, H))
    inv = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    s = rng.standard_normal((T, H))
    r = rng.standard_normal((T, H)).astype(np.float16)
    gt = np.array([0.5, 0.25, 0.0, 1.0, 0.8125])
    out, o64 = O.combine(y, inv, w, s, r, shared_gate=gt)
    out2, o642 = O.combine(y, inv, w, gt[:, None] * s, r)
    assert np.array_equal(o64, o642) and np.array_equal(out, out2)
    _, none64 = O.combine(y, inv, w, None, r)
    _, full64 = O.combine(y, inv, w, s, r)
    assert np.array_equal(o64[2], none64[2])
    assert np.array_equal(o64[3], full64[3])


def test_gated_layer_is_routed_plus_gate_times_dense_shared():
    cfg = MI.TINY
    T = 4
    x = MI.gen_x(cfg, T)
    wr = MI.gen_router(cfg)
    blobs = [O.pack_expert(*MI.gen_expert(cfg, 0, e), cfg.g) for e in range(cfg.E)]
    rng = np.random.default_rng(3)
    Is = 128
    sh = tuple(rng.normal(0, 0.02, sz).astype(np.float16)
               for sz in ((Is, cfg.H), (Is, cfg.H), (cfg.H, Is)))
    wsg = rng.normal(0, 0.05, cfg.H).astype(np.float16)
    r = O.moe_layer(x, wr, blobs, cfg.H, cfg.I, cfg.E, cfg.k, cfg.g, shared=sh,
                    shared_gate_w=wsg)
    r0 = O.moe_layer(x, wr, blobs, cfg.H, cfg.I, cfg.E, cfg.k, cfg.g)
    xs = x.astype(np.float64)
    dense = _dense_swiglu(xs, *(a.astype(np.float64) for a in sh))
    gate = 1.0 / (1.0 + np.exp(-(xs @ wsg.astype(np.float64))))
    assert np.allclose(r["out_f64"], r0["out_f64"] + gate[:, None] * dense, rtol=1e-11,
                       atol=1e-13)


# -------------------------------------------------------- threads, coverage

def test_thread_count_does_not_change_results():
    """The per-row loops spread rows over threads; every row keeps its own
    order of operations, so one thread and several give identical bits."""
    cfg = MI.MoEConfig(97, "thr", H=256, E=8, k=2, I=128, g=64)
    T = 37
    x = MI.gen_x(cfg, T)
    wr = MI.gen_router(cfg)
    blobs = [O.pack_expert(*MI.gen_expert(cfg, 0, e), cfg.g) for e in range(cfg.E)]
    wsh = tuple((np.random.default_rng(5).standard_normal(s) * 0.02).astype(np.float16)
                for s in ((64, cfg.H), (64, cfg.H), (cfg.H, 64)))
    outs = []
    try:
        for n in (1, 4):
            O.set_threads(n)
            r = O.moe_layer(x, wr, blobs, cfg.H, cfg.I, cfg.E, cfg.k, cfg.g, shared=wsh)
            outs.append(r)
    finally:
        O.set_threads(0)
    for key in ("idx", "w", "logits", "perm", "y", "shared", "out_f64"):
        assert np.array_equal(np.asarray(outs[0][key]).view(np.uint8),
                              np.asarray(outs[1][key]).view(np.uint8)), key


def _distinct_moments(E, k, n):
    """Exact mean and variance of the number of distinct experts touched by n
    tokens that each pick a uniformly random set of k distinct experts."""
    p0 = (1.0 - k / E) ** n                                   # one expert untouched
    p00 = ((E - k) * (E - k - 1) / (E * (E - 1))) ** n if E > 1 else 0.0   # two untouched
    mean = E * (1.0 - p0)
    var = E * p0 * (1.0 - p0) + E * (E - 1) * (p00 - p0 * p0)
    return mean, var


@pytest.mark.parametrize("E,k,n", [(64, 8, 1), (64, 8, 4), (64, 8, 16), (512, 10, 30),
                                   (8, 2, 5), (60, 4, 12)])
def test_coverage_of_uniform_traces(E, k, n):
    """Coverage formula of the local-inference explainer (step 3, how many
    experts a prompt touches): with uniform ("hash") routing, n tokens touch
    E (1 - (1 - k/E)^n) distinct experts on average.  Uniform routing is made
    through the oracle's own router: zero activations and router weights and a
    fresh iid fp32 bias per token, so the top-k of each token is a uniformly
    random k-subset (exchangeable logits, ties of probability ~0); the
    distinct count is the number of non-empty buckets of the oracle's
    permutation.  The trial mean must lie within 3 standard errors."""
    H = 8
    trials = 150
    rng = np.random.default_rng(E * 1000 + k * 10 + n)
    x = np.zeros((1, H), np.float16)
    wr = np.zeros((E, H), np.float16)
    d = []
    for _ in range(trials):
        idx = np.concatenate([O.route(x, wr, rng.standard_normal(E).astype(np.float32), k)[0]
                              for _ in range(n)])
        counts, _, _, _ = O.permute(idx, E)
        dt = int((counts > 0).sum())
        assert k <= dt <= min(E, n * k)
        d.append(dt)
    mean, var = _distinct_moments(E, k, n)
    se = math.sqrt(max(var, 0.0) / trials)
    assert abs(np.mean(d) - mean) <= 3 * se + 1e-9, (np.mean(d), mean, se)
    if n == 1:
        assert all(v == k for v in d)


def test_coverage_moments_brute_force():
    """The closed-form moments above against exhaustive enumeration on a tiny
    case (E = 5, k = 2, n = 3: every sequence of 2-subsets)."""
    E, k, n = 5, 2, 3
    subsets = list(itertools.combinations(range(E), k))
    vals = [len(set().union(*seq)) for seq in itertools.product(subsets, repeat=n)]
    mean, var = _distinct_moments(E, k, n)
    assert math.isclose(np.mean(vals), mean, rel_tol=1e-12)
    assert math.isclose(np.var(vals), var, rel_tol=1e-12)
