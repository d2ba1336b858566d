"""ctypes wrapper of the plain C CPU oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; the product package never
imports it.  All arrays are numpy; fp16 data travels as float16 arrays viewed
as uint16.  Every function forwards to the C routine of the same name, which
documents the passage of the pages (or the reading) it implements.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        L = C.CDLL(path)
        vp, i32, i64 = C.c_void_p, C.c_int, C.c_int64
        L.oracle_f16_to_f64.restype = C.c_double
        L.oracle_f16_to_f64.argtypes = [C.c_uint16]
        L.oracle_f64_to_f16.restype = C.c_uint16
        L.oracle_f64_to_f16.argtypes = [C.c_double]
        L.oracle_f16_to_f64_n.argtypes = [vp, vp, i64]
        L.oracle_f64_to_f16_n.argtypes = [vp, vp, i64]
        L.oracle_blob_layout.argtypes = [i32, i32, i32, vp, vp]
        L.oracle_quantize_rows.argtypes = [vp, i32, i32, i32, vp, vp]
        L.oracle_pack_expert.argtypes = [vp, vp, vp, i32, i32, i32, vp]
        L.oracle_dequant_rows.argtypes = [vp, vp, i32, i32, i32, vp]
        L.oracle_route.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]
        L.oracle_permute.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
        L.oracle_expert_ffn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                        vp, i32, vp]
        L.oracle_shared_ffn.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, i32, vp]
        L.oracle_shared_gate.argtypes = [vp, vp, i32, i32, vp, i32, vp]
        L.oracle_combine.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp]
        L.oracle_pool_sim.argtypes = [i32, i32, i32, i32, i32, vp, vp, i32, vp, vp, vp, vp]
        L.oracle_profile_pin.argtypes = [vp, i32, i32, i32, vp]
        L.oracle_pool_sim_pinned.argtypes = [i32, i32, i32, vp, i32, vp, vp, i32, vp, vp, vp]
        L.oracle_blob_layout_zp.argtypes = [i32, i32, i32, vp, vp]
        L.oracle_quantize_rows_zp.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.oracle_pack_expert_zp.argtypes = [vp, vp, vp, i32, i32, i32, vp]
        L.oracle_dequant_rows_zp.argtypes = [vp, vp, vp, i32, i32, i32, vp]
        L.oracle_expert_ffn_fmt.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                            vp, i32, vp]
        L.oracle_set_threads.argtypes = [i32]
        L.oracle_set_threads.restype = None
        L.oracle_get_threads.argtypes = []
        L.oracle_get_threads.restype = i32
        for name in ("oracle_blob_layout", "oracle_quantize_rows", "oracle_pack_expert",
                     "oracle_dequant_rows", "oracle_route", "oracle_permute",
                     "oracle_expert_ffn", "oracle_shared_ffn", "oracle_shared_gate",
                     "oracle_combine",
                     "oracle_pool_sim", "oracle_profile_pin", "oracle_pool_sim_pinned",
                     "oracle_blob_layout_zp", "oracle_quantize_rows_zp", "oracle_pack_expert_zp",
                     "oracle_dequant_rows_zp", "oracle_expert_ffn_fmt"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError("%s failed with code %d" % (what, rc))


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16
    return a


# ---------------------------------------------------------------- threads

def set_threads(n: int) -> None:
    """Worker threads of the per-row loops (route, expert FFN, shared FFN);
    n <= 0 restores the OpenMP default.  Results do not depend on it."""
    lib().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(lib().oracle_get_threads())


# ------------------------------------------------------------------- fp16

def f16_to_f64(bits) -> np.ndarray:
    bits = _u16(np.asarray(bits))
    out = np.empty(bits.shape, np.float64)
    lib().oracle_f16_to_f64_n(_p(bits), _p(out), bits.size)
    return out


def f64_to_f16(v) -> np.ndarray:
    """Round to fp16 (RNE); returns the bits as uint16."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_f64_to_f16_n(_p(v), _p(out), v.size)
    return out


# ------------------------------------------------------- blob & quantiser

FMT_SYM, FMT_ZP = 0, 1   # blob formats: symmetric (z = 8), zero point per group


def blob_layout(H, I, g, fmt=FMT_SYM):
    """Section offsets (6 symmetric, 9 with zero points) and total bytes."""
    n = 9 if fmt == FMT_ZP else 6
    off = np.zeros(n, np.int64)
    tot = np.zeros(1, np.int64)
    f = lib().oracle_blob_layout_zp if fmt == FMT_ZP else lib().oracle_blob_layout
    _check(f(H, I, g, _p(off), _p(tot)), "blob_layout")
    return [int(o) for o in off], int(tot[0])


def quantize_rows(w, g):
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, K = w.shape
    q = np.empty((rows, K // 2), np.uint8)
    s = np.empty((rows, K // g), np.uint16)
    _check(lib().oracle_quantize_rows(_p(w), rows, K, g, _p(q), _p(s)), "quantize_rows")
    return q, s


def quantize_rows_zp(w, g):
    """Zero-point quantiser: codes u [rows, K/2] u8, scales [rows, K/g] fp16
    bits, zero points [rows, K/g] u8."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, K = w.shape
    q = np.empty((rows, K // 2), np.uint8)
    s = np.empty((rows, K // g), np.uint16)
    z = np.empty((rows, K // g), np.uint8)
    _check(lib().oracle_quantize_rows_zp(_p(w), rows, K, g, _p(q), _p(s), _p(z)),
           "quantize_rows_zp")
    return q, s, z


def pack_expert(wg, wu, wd, g, fmt=FMT_SYM):
    wg = np.ascontiguousarray(wg, dtype=np.float32)
    wu = np.ascontiguousarray(wu, dtype=np.float32)
    wd = np.ascontiguousarray(wd, dtype=np.float32)
    I, H = wg.shape
    _, tot = blob_layout(H, I, g, fmt)
    blob = np.empty(tot, np.uint8)
    f = lib().oracle_pack_expert_zp if fmt == FMT_ZP else lib().oracle_pack_expert
    _check(f(_p(wg), _p(wu), _p(wd), H, I, g, _p(blob)), "pack_expert")
    return blob


def dequant_rows(q, s, g):
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = _u16(s)
    rows, K2 = q.shape
    out = np.empty((rows, 2 * K2), np.float64)
    _check(lib().oracle_dequant_rows(_p(q), _p(s), rows, 2 * K2, g, _p(out)), "dequant_rows")
    return out


def dequant_rows_zp(q, s, z, g):
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = _u16(s)
    z = np.ascontiguousarray(z, dtype=np.uint8)
    rows, K2 = q.shape
    out = np.empty((rows, 2 * K2), np.float64)
    _check(lib().oracle_dequant_rows_zp(_p(q), _p(s), _p(z), rows, 2 * K2, g, _p(out)),
           "dequant_rows_zp")
    return out


def blob_sections(blob, H, I, g, fmt=FMT_SYM):
    """Views (gate_q, up_q, down_q, gate_s, up_s, down_s[, gate_z, up_z,
    down_z]) of a canonical blob."""
    off, _ = blob_layout(H, I, g, fmt)
    gq = blob[off[0]:off[0] + I * H // 2].reshape(I, H // 2)
    uq = blob[off[1]:off[1] + I * H // 2].reshape(I, H // 2)
    dq = blob[off[2]:off[2] + H * I // 2].reshape(H, I // 2)
    gs = blob[off[3]:off[3] + I * (H // g) * 2].view(np.uint16).reshape(I, H // g)
    us = blob[off[4]:off[4] + I * (H // g) * 2].view(np.uint16).reshape(I, H // g)
    ds = blob[off[5]:off[5] + H * (I // g) * 2].view(np.uint16).reshape(H, I // g)
    if fmt != FMT_ZP:
        return gq, uq, dq, gs, us, ds
    gz = blob[off[6]:off[6] + I * (H // g)].reshape(I, H // g)
    uz = blob[off[7]:off[7] + I * (H // g)].reshape(I, H // g)
    dz = blob[off[8]:off[8] + H * (I // g)].reshape(H, I // g)
    return gq, uq, dq, gs, us, ds, gz, uz, dz


# ------------------------------------------------------------ layer steps

def route(x, wr, bias=None, k=1, renorm=False):
    x = _u16(x)
    wr = _u16(wr)
    T, H = x.shape
    E = wr.shape[0]
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    logits = np.empty((T, E), np.float32)
    _check(lib().oracle_route(_p(x), _p(wr), _p(b), T, H, E, k, int(renorm),
                              _p(idx), _p(w), _p(logits)), "route")
    return idx, w, logits


def permute(idx, E):
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv = np.empty(T * k, np.int32)
    _check(lib().oracle_permute(_p(idx), T, k, E, _p(counts), _p(offsets), _p(perm), _p(inv)),
           "permute")
    return counts, offsets, perm, inv


def expert_ffn(x, perm, offsets, blobs, H, I, E, k, g, rows=None, fmt=FMT_SYM):
    """y[len(rows) or T*k, H] fp64 for the selected sorted rows.  `blobs` is a
    list of E canonical blobs (numpy uint8) or None for experts not needed;
    fmt is their format (FMT_SYM or FMT_ZP)."""
    x = _u16(x)
    T = x.shape[0]
    perm = np.ascontiguousarray(perm, dtype=np.int32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    ptrs = (C.c_void_p * E)(*[None if b is None else b.ctypes.data for b in blobs])
    if rows is None:
        r = None
        n = T * k
    else:
        r = np.ascontiguousarray(rows, dtype=np.int32)
        n = r.size
    y = np.empty((n, H), np.float64)
    _check(lib().oracle_expert_ffn_fmt(_p(x), _p(perm), _p(offsets), C.cast(ptrs, C.c_void_p),
                                       T, H, I, E, k, g, int(fmt), _p(r), n, _p(y)),
           "expert_ffn")
    return y


def shared_ffn(x, wg, wu, wd, toks=None):
    x = _u16(x)
    wg, wu, wd = _u16(wg), _u16(wu), _u16(wd)
    T, H = x.shape
    Is = wg.shape[0]
    if toks is None:
        tk, n = None, T
    else:
        tk = np.ascontiguousarray(toks, dtype=np.int32)
        n = tk.size
    s = np.empty((n, H), np.float64)
    _check(lib().oracle_shared_ffn(_p(x), _p(wg), _p(wu), _p(wd), T, H, Is, _p(tk), n, _p(s)),
           "shared_ffn")
    return s


def shared_gate(x, wsg, toks=None):
    """Per-token sigmoid gate of the shared expert, fp64 [ntoks]."""
    x = _u16(x)
    wsg = _u16(wsg).reshape(-1)
    T, H = x.shape
    assert wsg.size == H
    if toks is None:
        tk, n = None, T
    else:
        tk = np.ascontiguousarray(toks, dtype=np.int32)
        n = tk.size
    gt = np.empty(n, np.float64)
    _check(lib().oracle_shared_gate(_p(x), _p(wsg), T, H, _p(tk), n, _p(gt)), "shared_gate")
    return gt


def combine(y, inv_perm, w, shared=None, residual=None, shared_gate=None):
    """Returns (out fp16 as np.float16 [T,H], pre-rounding fp64 value).
    shared_gate (fp64 [T]) scales the shared rows when given."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    inv = np.ascontiguousarray(inv_perm, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, k = w.shape
    H = y.shape[1]
    sh = None if shared is None else np.ascontiguousarray(shared, dtype=np.float64)
    res = None if residual is None else _u16(residual)
    gt = None if shared_gate is None else np.ascontiguousarray(shared_gate, dtype=np.float64)
    assert gt is None or (sh is not None and gt.size == T)
    out = np.empty((T, H), np.uint16)
    o64 = np.empty((T, H), np.float64)
    _check(lib().oracle_combine(_p(y), _p(inv), _p(w), _p(sh), _p(gt), _p(res), T, H, k,
                                _p(out), _p(o64)), "combine")
    return out.view(np.float16), o64


def pool_sim(L, E, C_, shift, k, ev_layer, ev_ids):
    ev_layer = np.ascontiguousarray(ev_layer, dtype=np.int32)
    ev_ids = np.ascontiguousarray(ev_ids, dtype=np.int32).reshape(-1, k)
    n = ev_layer.size
    hits = np.empty(n, np.int32)
    misses = np.empty(n, np.int32)
    ml = np.empty((n, k), np.int32)
    el = np.empty((n, k), np.int32)
    _check(lib().oracle_pool_sim(L, E, C_, shift, k, _p(ev_layer), _p(ev_ids), n,
                                 _p(hits), _p(misses), _p(ml), _p(el)), "pool_sim")
    return hits, misses, ml, el


def profile_pin(counts, C):
    """counts [L, E] int64 routed-event counts -> pinned [L, C] int32 (the C
    most counted experts per layer, ties to the lower id, ascending id)."""
    counts = np.ascontiguousarray(counts, dtype=np.int64)
    L_, E = counts.shape
    pinned = np.empty((L_, C), np.int32)
    _check(lib().oracle_profile_pin(_p(counts), L_, E, C, _p(pinned)), "profile_pin")
    return pinned


def pool_sim_pinned(L, E, pinned, k, ev_layer, ev_ids):
    """Replays events through the pinned policy: (hits, misses, miss_list)."""
    pinned = np.ascontiguousarray(pinned, dtype=np.int32)
    C_ = pinned.shape[1]
    ev_layer = np.ascontiguousarray(ev_layer, dtype=np.int32)
    ev_ids = np.ascontiguousarray(ev_ids, dtype=np.int32).reshape(-1, k)
    n = ev_layer.size
    hits = np.empty(n, np.int32)
    misses = np.empty(n, np.int32)
    ml = np.empty((n, k), np.int32)
    _check(lib().oracle_pool_sim_pinned(L, E, C_, _p(pinned), k, _p(ev_layer), _p(ev_ids), n,
                                        _p(hits), _p(misses), _p(ml)), "pool_sim_pinned")
    return hits, misses, ml


def moe_layer(x, wr, blobs, H, I, E, k, g, bias=None, renorm=False,
              shared=None, residual=None, shared_gate_w=None, fmt=FMT_SYM):
    """The whole layer in the oracle: route, permute, expert FFN (all rows),
    optional shared FFN (optionally gated), combine.  Returns a dict of every
    intermediate."""
    idx, w, logits = route(x, wr, bias, k, renorm)
    counts, offsets, perm, inv = permute(idx, E)
    y = expert_ffn(x, perm, offsets, blobs, H, I, E, k, g, fmt=fmt)
    s = None if shared is None else shared_ffn(x, *shared)
    gt = None if shared_gate_w is None else shared_gate(x, shared_gate_w)
    out, o64 = combine(y, inv, w, s, residual, gt)
    return dict(idx=idx, w=w, logits=logits, counts=counts, offsets=offsets, perm=perm,
                inv_perm=inv, y=y, shared=s, gate=gt, out=out, out_f64=o64)
