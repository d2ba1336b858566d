"""Pins of the oracle's zero-point (asymmetric) INT4 format, against facts
that do not come from the oracle: the closed-form round-trip bound of the
min/max affine rule, exact round trips of weights the format represents, the
byte layout, the symmetric format as the case z = 8, and a single-expert
layer equal to a dense SwiGLU FFN written here in numpy.

Source: the local-inference explainer's step 1 (every block of weights
carries a scale and a zero point); the rule itself is a stated reading."""
import numpy as np
import pytest

import moe_inputs as MI
import oracle as O


def _al(x):
    return (x + 255) // 256 * 256


def _codes(q):
    out = np.empty((q.shape[0], q.shape[1] * 2), np.int64)
    out[:, 0::2] = q & 15
    out[:, 1::2] = q >> 4
    return out


@pytest.mark.parametrize("g", [32, 64, 128])
def test_zp_round_trip_bound_closed_form(g):
    """|w - (u - z) s| <= s/2 + 15 |s - s*| for every element, s* the exact
    (hi - lo) / 15: inside the grid the error is half a step; at a clamped end
    it also absorbs the scale's fp16 rounding (15 steps of |s - s*|)."""
    rng = np.random.default_rng(g)
    rows, K = 96, 1024
    w = rng.standard_normal((rows, K)).astype(np.float32) * np.float32(0.02)
    # skewed groups too: all positive, all negative, mostly positive
    w[10] = np.abs(w[10])
    w[11] = -np.abs(w[11])
    w[12] = w[12] + np.float32(0.03)
    q, s, z = O.quantize_rows_zp(w, g)
    u = _codes(q)
    assert u.min() >= 0 and u.max() <= 15 and z.max() <= 15
    sv = s.view(np.float16).astype(np.float64)
    wg = w.astype(np.float64).reshape(rows, K // g, g)
    lo = np.minimum(wg.min(axis=2), 0.0)
    hi = np.maximum(wg.max(axis=2), 0.0)
    sstar = (hi - lo) / 15.0
    assert np.all(np.abs(sv - sstar) <= sstar * 2.0 ** -11 + 1e-12)   # fp16 rounding of s
    deq = (u.reshape(rows, K // g, g) - z[:, :, None].astype(np.int64)) * sv[:, :, None]
    bound = sv / 2 + 15 * np.abs(sv - sstar) + 1e-6 * sv
    assert np.all(np.abs(wg - deq) <= bound[:, :, None])
    # the oracle's own dequantiser agrees with (u - z) s computed here
    assert np.array_equal(O.dequant_rows_zp(q, s, z, g), deq.reshape(rows, K))
    # all-positive / all-negative groups keep zero inside: z = 0 / z = 15
    assert np.all(z[10] == 0) and np.all(z[11] == 15)


def test_zp_exact_round_trip_of_representable_weights():
    """w = (u - z) 2^-m with u spanning 0..15 in every group: s = 2^-m and z
    are recovered exactly, and so are the codes and the weights."""
    rng = np.random.default_rng(7)
    g, rows, K = 64, 32, 512
    ng = K // g
    m = rng.integers(6, 12, (rows, ng))
    zz = rng.integers(0, 16, (rows, ng))
    uu = rng.integers(0, 16, (rows, ng, g))
    uu[:, :, 0] = 0
    uu[:, :, 1] = 15
    w = ((uu - zz[:, :, None]) * (2.0 ** -m)[:, :, None]).astype(np.float32).reshape(rows, K)
    q, s, z = O.quantize_rows_zp(w, g)
    assert np.array_equal(z.astype(np.int64), zz)
    assert np.array_equal(s.view(np.float16).astype(np.float64), 2.0 ** -m)
    assert np.array_equal(_codes(q), uu.reshape(rows, K))
    assert np.array_equal(O.dequant_rows_zp(q, s, z, g), w.astype(np.float64))


def test_zp_zero_group_and_symmetric_case():
    """An all-zero group has s = 0, z = 0, u = 0; and the zero-point decoder
    with z = 8 is the symmetric decoder of the same codes and scales."""
    g = 32
    w = np.zeros((2, 64), np.float32)
    w[1, 32:] = np.linspace(-1, 1, 32, dtype=np.float32)
    q, s, z = O.quantize_rows_zp(w, g)
    assert s[0, 0] == 0 and z[0, 0] == 0 and np.all(q[0] == 0) and s[1, 0] == 0
    assert np.all(O.dequant_rows_zp(q, s, z, g)[0] == 0.0)
    rng = np.random.default_rng(3)
    qs, ss = O.quantize_rows(rng.standard_normal((8, 256)).astype(np.float32), g)
    z8 = np.full(ss.shape, 8, np.uint8)
    assert np.array_equal(O.dequant_rows_zp(qs, ss, z8, g), O.dequant_rows(qs, ss, g))


@pytest.mark.parametrize("H,I,g", [(256, 512, 64), (2048, 1024, 128), (512, 192, 32)])
def test_zp_blob_layout_closed_form(H, I, g):
    """Nine sections: the six of the symmetric blob at the same offsets, then
    one zero-point byte per group of each projection, 256-byte aligned."""
    off6, tot6 = O.blob_layout(H, I, g)
    off9, tot9 = O.blob_layout(H, I, g, O.FMT_ZP)
    assert off9[:6] == off6
    assert off9[6] == tot6
    assert off9[7] == off9[6] + _al(I * (H // g))
    assert off9[8] == off9[7] + _al(I * (H // g))
    assert tot9 == off9[8] + _al(H * (I // g))
    cfg = MI.MoEConfig(80, "zp", H=H, E=1, k=1, I=I, g=g)
    wg, wu, wd = MI.gen_expert(cfg, 0, 0)
    blob = O.pack_expert(wg, wu, wd, g, O.FMT_ZP)
    gq, uq, dq, gs, us, ds, gz, uz, dz = O.blob_sections(blob, H, I, g, O.FMT_ZP)
    for w_, q_, s_, z_ in ((wg, gq, gs, gz), (wu, uq, us, uz), (wd, dq, ds, dz)):
        q2, s2, z2 = O.quantize_rows_zp(w_, g)
        assert np.array_equal(q_, q2) and np.array_equal(s_, s2) and np.array_equal(z_, z2)


def test_zp_single_expert_layer_equals_dense_swiglu():
    """E = 1, k = 1 (weight exactly 1): the layer output with a zero-point blob
    equals a dense SwiGLU FFN on the dequantised matrices, computed here."""
    cfg = MI.MoEConfig(81, "zp_e1", H=256, E=1, k=1, I=128, g=64)
    T = 9
    wg, wu, wd = MI.gen_expert(cfg, 0, 0)
    blob = O.pack_expert(wg, wu, wd, cfg.g, O.FMT_ZP)
    x = MI.gen_x(cfg, T)
    wr = MI.gen_router(cfg)
    ref = O.moe_layer(x, wr, [blob], cfg.H, cfg.I, cfg.E, cfg.k, cfg.g, fmt=O.FMT_ZP)
    assert np.all(ref["w"] == 1.0)

    def dense(w_):
        q, s, z = O.quantize_rows_zp(w_, cfg.g)
        u = _codes(q)
        zz = np.repeat(z.astype(np.int64), cfg.g, axis=1)
        return (u - zz) * np.repeat(s.view(np.float16).astype(np.float64), cfg.g, axis=1)

    Wg, Wu, Wd = dense(wg), dense(wu), dense(wd)
    xv = x.astype(np.float64)
    a, u = xv @ Wg.T, xv @ Wu.T
    y = ((a / (1.0 + np.exp(-a))) * u) @ Wd.T
    assert np.allclose(ref["out_f64"], y, rtol=0, atol=1e-12 * max(1.0, np.abs(y).max()))
    # and the zero-point FFN is not the symmetric one of the same weights
    sym = O.moe_layer(x, wr, [O.pack_expert(wg, wu, wd, cfg.g)], cfg.H, cfg.I, cfg.E, cfg.k,
                      cfg.g)
    assert not np.array_equal(sym["out_f64"], ref["out_f64"])
