"""ctypes marshalling for libmoe_w4a16.so (see include/moe_w4a16.h)."""
from __future__ import annotations

import ctypes as C
import os

from . import build as _build

__all__ = [
    "MoEError", "lib", "MOE_OK", "MOE_EINVAL", "MOE_EUNSUPPORTED", "MOE_ENOMEM", "MOE_EHIP",
    "MOE_ECAPACITY", "MOE_ESTATE", "MOE_RENORM", "MOE_REGIME_AUTO", "MOE_REGIME_DECODE",
    "MOE_REGIME_BATCHED", "MOE_REGIME_SMALL", "MOE_Y_TOKEN_ORDER", "MOE_Y_PARTIAL_ORDER",
    "MOE_DTYPE_F16", "MOE_DTYPE_F32", "MOE_DTYPE_F32_PM", "MOE_FMT_SYM", "MOE_FMT_ZP", "MOE_W4_ZERO_POINT", "EXPORTS",
    "moe_blob_layout_fmt", "moe_quantize_experts_fmt", "moe_prepack_experts_fmt",
    "moe_unpack_experts_fmt", "moe_prepack_expert_host", "moe_unpack_expert_host",
    "moe_last_error", "moe_workspace_clear", "moe_blob_layout", "moe_quantize_experts",
    "moe_prepack_experts",
    "moe_unpack_experts", "moe_route_workspace_bytes", "moe_route", "moe_permute_workspace_bytes",
    "moe_permute", "moe_route_permute_workspace_bytes", "moe_route_permute",
    "moe_route_permute_noalloc",
    "moe_expert_ffn_plan", "moe_expert_ffn_w4a16", "moe_shared_ffn_workspace_bytes",
    "moe_shared_ffn_f16", "moe_combine", "moe_combine_gated",
    "moe_combine_route_permute_workspace_bytes", "moe_combine_route_permute",
    "moe_logit_partials_bytes", "moe_logit_partials", "moe_combine_route_partials",
    "moe_expert_ffn_w4a16_routed",
    "PoolConfig",
    "PoolStats", "PoolLayerArgs",
    "moe_pool_create", "moe_pool_prepare", "moe_pool_layer_forward", "moe_pool_pin",
    "moe_pool_retire", "moe_pool_stats", "moe_pool_access_counts", "moe_pool_reset",
    "moe_pool_destroy",
]

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ENOMEM, MOE_EHIP, MOE_ECAPACITY, MOE_ESTATE = \
    0, -1, -2, -3, -4, -5, -6
MOE_RENORM = 1
MOE_REGIME_AUTO, MOE_REGIME_DECODE, MOE_REGIME_BATCHED, MOE_REGIME_SMALL = 0, 1, 2, 3
MOE_Y_TOKEN_ORDER = 0x100   # OR'd into a regime: decode y rows in token order
MOE_Y_PARTIAL_ORDER = 0x400  # OR'd into a regime: decode y columns in partial-major order
MOE_DTYPE_F16, MOE_DTYPE_F32, MOE_DTYPE_F32_PM = 0, 1, 2
MOE_FMT_SYM, MOE_FMT_ZP = 0, 1   # expert blob formats (zero point per group)
MOE_W4_ZERO_POINT = 0x200        # OR'd into a regime: the blobs are MOE_FMT_ZP

# every symbol include/moe_w4a16.h declares
EXPORTS = [
    "moe_blob_layout_fmt", "moe_quantize_experts_fmt", "moe_prepack_experts_fmt",
    "moe_unpack_experts_fmt", "moe_prepack_expert_host", "moe_unpack_expert_host",
    "moe_last_error", "moe_workspace_clear", "moe_blob_layout", "moe_quantize_experts",
    "moe_prepack_experts", "moe_unpack_experts", "moe_route_workspace_bytes", "moe_route", "moe_permute_workspace_bytes",
    "moe_permute", "moe_route_permute_workspace_bytes", "moe_route_permute",
    "moe_route_permute_noalloc",
    "moe_expert_ffn_plan", "moe_expert_ffn_w4a16", "moe_shared_ffn_workspace_bytes",
    "moe_shared_ffn_f16", "moe_combine", "moe_combine_gated",
    "moe_combine_route_permute_workspace_bytes", "moe_combine_route_permute",
    "moe_logit_partials_bytes", "moe_logit_partials", "moe_combine_route_partials",
    "moe_expert_ffn_w4a16_routed",
    "moe_pool_create",
    "moe_pool_prepare",
    "moe_pool_layer_forward", "moe_pool_pin",
    "moe_pool_retire", "moe_pool_stats", "moe_pool_access_counts", "moe_pool_reset",
    "moe_pool_destroy",
]


class MoEError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("moe error %d: %s" % (code, msg))
        self.code = code


class PoolConfig(C.Structure):
    _fields_ = [("layers", C.c_int), ("experts", C.c_int), ("topk", C.c_int),
                ("capacity", C.c_int), ("spares", C.c_int), ("decay_shift", C.c_int),
                ("expert_bytes", C.c_int64)]


class PoolStats(C.Structure):
    _fields_ = [("hits", C.c_int64), ("misses", C.c_int64), ("evictions", C.c_int64),
                ("h2d_bytes", C.c_int64), ("generation", C.c_int64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class PoolLayerArgs(C.Structure):
    """moe_pool_layer_args: device pointers as ints, host_ids a pinned host address."""
    _fields_ = [("x_f16", C.c_void_p), ("w_router_f16", C.c_void_p), ("logit_bias", C.c_void_p),
                ("T", C.c_int), ("H", C.c_int), ("I", C.c_int), ("k", C.c_int),
                ("group", C.c_int), ("flags", C.c_uint),
                ("topk_idx", C.c_void_p), ("topk_w", C.c_void_p), ("counts", C.c_void_p),
                ("offsets", C.c_void_p), ("perm", C.c_void_p), ("inv_perm", C.c_void_p),
                ("route_ws", C.c_void_p), ("route_ws_bytes", C.c_size_t),
                ("regime", C.c_int), ("y", C.c_void_p), ("y_dtype", C.c_int),
                ("y_slices", C.c_int), ("ffn_ws", C.c_void_p), ("ffn_ws_bytes", C.c_size_t),
                ("shared_f32", C.c_void_p), ("residual_f16", C.c_void_p),
                ("out_f16", C.c_void_p), ("host_ids", C.c_void_p)]


_lib = None
vp, i32, i64, sz = C.c_void_p, C.c_int, C.c_int64, C.c_size_t


def _declare(L):
    sig = {
        "moe_last_error": (C.c_char_p, []),
        "moe_workspace_clear": (i32, [vp, sz, vp]),
        "moe_blob_layout": (i32, [i32, i32, i32, vp, vp]),
        "moe_blob_layout_fmt": (i32, [i32, i32, i32, i32, vp, vp]),
        "moe_quantize_experts_fmt": (i32, [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]),
        "moe_prepack_experts_fmt": (i32, [vp, i32, i32, i32, i32, i32, vp, vp]),
        "moe_unpack_experts_fmt": (i32, [vp, i32, i32, i32, i32, i32, vp, vp]),
        "moe_prepack_expert_host": (i32, [vp, i32, i32, i32, i32, vp]),
        "moe_unpack_expert_host": (i32, [vp, i32, i32, i32, i32, vp]),
        "moe_quantize_experts": (i32, [vp, vp, vp, i32, i32, i32, i32, vp, vp]),
        "moe_prepack_experts": (i32, [vp, i32, i32, i32, i32, vp, vp]),
        "moe_unpack_experts": (i32, [vp, i32, i32, i32, i32, vp, vp]),
        "moe_route_workspace_bytes": (sz, [i32, i32]),
        "moe_route": (i32, [vp, vp, vp, i32, i32, i32, i32, C.c_uint, vp, vp, vp, sz, vp]),
        "moe_permute_workspace_bytes": (sz, [i32, i32, i32]),
        "moe_permute": (i32, [vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
        "moe_route_permute_workspace_bytes": (sz, [i32, i32, i32]),
        "moe_route_permute": (i32, [vp, vp, vp, i32, i32, i32, i32, C.c_uint, vp, vp, vp, vp,
                                    vp, vp, vp, sz, vp]),
        "moe_route_permute_noalloc": (i32, [vp, vp, vp, i32, i32, i32, i32, C.c_uint, vp, vp,
                                            vp, vp, vp, vp, vp]),
        "moe_expert_ffn_plan": (i32, [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp]),
        "moe_expert_ffn_w4a16": (i32, [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                       vp, i32, i32, vp, sz, vp]),
        "moe_shared_ffn_workspace_bytes": (sz, [i32, i32, i32]),
        "moe_shared_ffn_f16": (i32, [vp, vp, vp, vp, i32, i32, i32, vp, vp, sz, vp]),
        "moe_combine": (i32, [vp, i32, i32, vp, vp, vp, vp, i32, i32, i32, vp, vp]),
        "moe_combine_gated": (i32, [vp, i32, i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, vp,
                                    vp]),
        "moe_combine_route_permute_workspace_bytes": (sz, [i32, i32, i32]),
        "moe_combine_route_permute": (i32, [vp, i32, i32, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                            vp, vp, vp, i32, i32, C.c_uint, vp, vp, vp, vp, vp,
                                            vp, vp, sz, vp]),
        "moe_logit_partials_bytes": (sz, []),
        "moe_logit_partials": (i32, [vp, vp, i32, i32, i32, vp, vp]),
        "moe_combine_route_partials": (i32, [vp, i32, i32, vp, vp, vp, vp, vp, vp, i32, i32,
                                             i32, vp, vp, i32, vp, vp]),
        "moe_expert_ffn_w4a16_routed": (i32, [vp, vp, vp, i32, i32, C.c_uint, vp, vp, vp, vp,
                                              vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, i32,
                                              vp]),
        "moe_pool_create": (i32, [C.POINTER(PoolConfig), vp, C.POINTER(vp)]),
        "moe_pool_prepare": (i32, [vp, i32, vp, i32, vp, C.POINTER(vp), C.POINTER(PoolStats)]),
        "moe_pool_layer_forward": (i32, [vp, i32, C.POINTER(PoolLayerArgs), vp,
                                         C.POINTER(PoolStats)]),
        "moe_pool_pin": (i32, [vp, i32, vp, i32]),
        "moe_pool_retire": (i32, [vp, i32, vp]),
        "moe_pool_stats": (i32, [vp, C.POINTER(PoolStats)]),
        "moe_pool_access_counts": (i32, [vp, vp, vp]),
        "moe_pool_reset": (i32, [vp]),
        "moe_pool_destroy": (i32, [vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args


def lib(path: str | None = None):
    """Load (building in-tree first if absent) libmoe_w4a16.so.

    torch is imported first: its wheel carries its own HIP runtime under the
    same soname, and loading torch first makes this library bind to that one
    copy instead of pulling in a second runtime."""
    global _lib
    if _lib is None:
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        path = path or _build.LIB
        if not os.path.exists(path):
            _build.build()
        _lib = C.CDLL(path)
        _declare(_lib)
    return _lib


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def _check(rc):
    if rc != 0:
        raise MoEError(rc, moe_last_error())
    return rc


def _p(t):
    """Device/host pointer of a tensor (or an int address); None -> NULL."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------- entries

def moe_workspace_clear(ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().moe_workspace_clear(_p(ws), ws_bytes, _s(stream)))


def moe_blob_layout(H, I, group):
    off = (C.c_int64 * 6)()
    tot = C.c_int64()
    _check(lib().moe_blob_layout(H, I, group, off, C.byref(tot)))
    return list(off), tot.value


def moe_blob_layout_fmt(H, I, group, fmt):
    off = (C.c_int64 * 9)()
    tot = C.c_int64()
    _check(lib().moe_blob_layout_fmt(H, I, group, fmt, off, C.byref(tot)))
    return list(off), tot.value


def moe_quantize_experts_fmt(wg, wu, wd, n, H, I, group, fmt, blobs, stream=None):
    _check(lib().moe_quantize_experts_fmt(_p(wg), _p(wu), _p(wd), n, H, I, group, fmt,
                                          _p(blobs), _s(stream)))


def moe_prepack_experts_fmt(src, n, H, I, group, fmt, dst, stream=None):
    _check(lib().moe_prepack_experts_fmt(_p(src), n, H, I, group, fmt, _p(dst), _s(stream)))


def moe_unpack_experts_fmt(src, n, H, I, group, fmt, dst, stream=None):
    _check(lib().moe_unpack_experts_fmt(_p(src), n, H, I, group, fmt, _p(dst), _s(stream)))


def moe_prepack_expert_host(src, H, I, group, fmt, dst):
    """One canonical blob to the device layout on the host (numpy uint8 arrays,
    or host addresses as ints)."""
    _check(lib().moe_prepack_expert_host(_hp(src), H, I, group, fmt, _hp(dst)))


def moe_unpack_expert_host(src, H, I, group, fmt, dst):
    _check(lib().moe_unpack_expert_host(_hp(src), H, I, group, fmt, _hp(dst)))


def _hp(a):
    """Host address of a numpy array (or an int address)."""
    if isinstance(a, int):
        return a
    if hasattr(a, "ctypes"):
        return a.ctypes.data
    return a.data_ptr()


def moe_quantize_experts(wg, wu, wd, n, H, I, group, blobs, stream=None):
    return _check(lib().moe_quantize_experts(_p(wg), _p(wu), _p(wd), n, H, I, group, _p(blobs),
                                             _s(stream)))


def moe_prepack_experts(src, n, H, I, group, dst, stream=None):
    return _check(lib().moe_prepack_experts(_p(src), n, H, I, group, _p(dst), _s(stream)))


def moe_unpack_experts(src, n, H, I, group, dst, stream=None):
    return _check(lib().moe_unpack_experts(_p(src), n, H, I, group, _p(dst), _s(stream)))


def moe_route_workspace_bytes(T, E):
    return lib().moe_route_workspace_bytes(T, E)


def moe_route(x, w_router, logit_bias, T, H, E, k, flags, topk_idx, topk_w, ws=None, ws_bytes=0,
              stream=None):
    return _check(lib().moe_route(_p(x), _p(w_router), _p(logit_bias), T, H, E, k, flags,
                                  _p(topk_idx), _p(topk_w), _p(ws), ws_bytes, _s(stream)))


def moe_permute_workspace_bytes(T, k, E):
    return lib().moe_permute_workspace_bytes(T, k, E)


def moe_permute(topk_idx, T, k, E, counts, offsets, perm, inv_perm, ws=None, ws_bytes=0,
                stream=None):
    return _check(lib().moe_permute(_p(topk_idx), T, k, E, _p(counts), _p(offsets), _p(perm),
                                    _p(inv_perm), _p(ws), ws_bytes, _s(stream)))


def moe_route_permute_workspace_bytes(T, k, E):
    return lib().moe_route_permute_workspace_bytes(T, k, E)


def moe_route_permute(x, w_router, logit_bias, T, H, E, k, flags, topk_idx, topk_w, counts,
                      offsets, perm, inv_perm, ws=None, ws_bytes=0, stream=None):
    return _check(lib().moe_route_permute(_p(x), _p(w_router), _p(logit_bias), T, H, E, k,
                                          flags, _p(topk_idx), _p(topk_w), _p(counts),
                                          _p(offsets), _p(perm), _p(inv_perm), _p(ws), ws_bytes,
                                          _s(stream)))


def moe_route_permute_noalloc(x, w_router, logit_bias, T, H, E, k, flags, topk_idx, topk_w,
                              counts, offsets, perm, inv_perm, stream=None):
    _check(lib().moe_route_permute_noalloc(_p(x), _p(w_router), _p(logit_bias), T, H, E, k,
                                           flags, _p(topk_idx), _p(topk_w), _p(counts),
                                           _p(offsets), _p(perm), _p(inv_perm), _s(stream)))


def moe_expert_ffn_plan(T, H, I, E, k, group, regime=MOE_REGIME_AUTO):
    """Returns (resolved_regime, y_dtype, y_slices, ws_bytes)."""
    r, dt, sl, ws = C.c_int(), C.c_int(), C.c_int(), C.c_size_t()
    _check(lib().moe_expert_ffn_plan(T, H, I, E, k, group, regime, C.byref(r), C.byref(dt),
                                     C.byref(sl), C.byref(ws)))
    return r.value, dt.value, sl.value, ws.value


def moe_expert_ffn_w4a16(x, perm, offsets, d_expert_blobs, T, H, I, E, k, group, regime, y,
                         y_dtype, y_slices, ws=None, ws_bytes=0, stream=None):
    return _check(lib().moe_expert_ffn_w4a16(
        _p(x), _p(perm), _p(offsets), _p(d_expert_blobs), T, H, I, E, k, group, regime, _p(y),
        y_dtype, y_slices, _p(ws), ws_bytes, _s(stream)))


def moe_shared_ffn_workspace_bytes(T, H, Is):
    return lib().moe_shared_ffn_workspace_bytes(T, H, Is)


def moe_shared_ffn_f16(x, wg, wu, wd, T, H, Is, out_f32, ws=None, ws_bytes=0, stream=None):
    return _check(lib().moe_shared_ffn_f16(_p(x), _p(wg), _p(wu), _p(wd), T, H, Is, _p(out_f32),
                                           _p(ws), ws_bytes, _s(stream)))


def moe_combine(y, y_dtype, y_slices, inv_perm, topk_w, shared_f32, residual_f16, T, H, k,
                out_f16, stream=None):
    return _check(lib().moe_combine(_p(y), y_dtype, y_slices, _p(inv_perm), _p(topk_w),
                                    _p(shared_f32), _p(residual_f16), T, H, k, _p(out_f16),
                                    _s(stream)))


def moe_combine_gated(y, y_dtype, y_slices, inv_perm, topk_w, shared_f32, x_f16, gate_w_f16,
                      residual_f16, T, H, k, out_f16, stream=None):
    return _check(lib().moe_combine_gated(_p(y), y_dtype, y_slices, _p(inv_perm), _p(topk_w),
                                          _p(shared_f32), _p(x_f16), _p(gate_w_f16),
                                          _p(residual_f16), T, H, k, _p(out_f16), _s(stream)))


def moe_combine_route_permute_workspace_bytes(T, k_next, E):
    return lib().moe_combine_route_permute_workspace_bytes(T, k_next, E)


def moe_combine_route_permute(y, y_dtype, y_slices, inv_perm, topk_w, shared_f32, x_f16,
                              gate_w_f16, residual_f16, T, H, k, out_f16, w_router, logit_bias,
                              E, k_next, flags, topk_idx, topk_w_next, counts, offsets, perm,
                              inv_perm_next, ws=None, ws_bytes=0, stream=None):
    return _check(lib().moe_combine_route_permute(
        _p(y), y_dtype, y_slices, _p(inv_perm), _p(topk_w), _p(shared_f32), _p(x_f16),
        _p(gate_w_f16), _p(residual_f16), T, H, k, _p(out_f16), _p(w_router), _p(logit_bias),
        E, k_next, flags, _p(topk_idx), _p(topk_w_next), _p(counts), _p(offsets), _p(perm),
        _p(inv_perm_next), _p(ws), ws_bytes, _s(stream)))


def moe_logit_partials_bytes():
    return lib().moe_logit_partials_bytes()


def moe_logit_partials(x_f16, w_router, T, H, E, logit_partials, stream=None):
    return _check(lib().moe_logit_partials(_p(x_f16), _p(w_router), T, H, E,
                                           _p(logit_partials), _s(stream)))


def moe_combine_route_partials(y, y_dtype, y_slices, inv_perm, topk_w, shared_f32, x_f16,
                               gate_w_f16, residual_f16, T, H, k, out_f16, w_router, E,
                               logit_partials, stream=None):
    return _check(lib().moe_combine_route_partials(
        _p(y), y_dtype, y_slices, _p(inv_perm), _p(topk_w), _p(shared_f32), _p(x_f16),
        _p(gate_w_f16), _p(residual_f16), T, H, k, _p(out_f16), _p(w_router), E,
        _p(logit_partials), _s(stream)))


def moe_expert_ffn_w4a16_routed(x, logit_partials, logit_bias, E, k, flags, topk_idx, topk_w,
                                counts, offsets, perm, inv_perm, d_expert_blobs, T, H, I, group,
                                regime, y, y_dtype, y_slices, stream=None):
    return _check(lib().moe_expert_ffn_w4a16_routed(
        _p(x), _p(logit_partials), _p(logit_bias), E, k, flags, _p(topk_idx), _p(topk_w),
        _p(counts), _p(offsets), _p(perm), _p(inv_perm), _p(d_expert_blobs), T, H, I, group,
        regime, _p(y), y_dtype, y_slices, _s(stream)))


def moe_pool_create(cfg: PoolConfig, pinned_src_ptrs):
    """pinned_src_ptrs: sequence of L*E host addresses (ints)."""
    arr = (C.c_void_p * len(pinned_src_ptrs))(*pinned_src_ptrs)
    h = C.c_void_p()
    _check(lib().moe_pool_create(C.byref(cfg), C.cast(arr, C.c_void_p), C.byref(h)))
    return h


def moe_pool_prepare(pool, layer, host_ids, n, compute=None):
    """host_ids: host address (int) or a numpy int32 array.  Returns
    (device table address, PoolStats of this step)."""
    if hasattr(host_ids, "ctypes"):
        host_ids = host_ids.ctypes.data
    tab = C.c_void_p()
    st = PoolStats()
    _check(lib().moe_pool_prepare(pool, layer, host_ids, n, _s(compute), C.byref(tab),
                                  C.byref(st)))
    return tab.value, st


def moe_pool_layer_forward(pool, layer, args: PoolLayerArgs, stream=None, step=None):
    """Runs one pooled layer (see PoolLayerArgs); returns this step's PoolStats
    (`step`, if given, is filled and returned)."""
    st = PoolStats() if step is None else step
    _check(lib().moe_pool_layer_forward(pool, layer, C.byref(args), _s(stream), C.byref(st)))
    return st


def moe_pool_pin(pool, layer, experts):
    """experts: host sequence of C distinct expert ids (the pinned set)."""
    import numpy as np
    ids = np.ascontiguousarray(experts, dtype=np.int32)
    return _check(lib().moe_pool_pin(pool, layer, ids.ctypes.data, ids.size))


def moe_pool_retire(pool, layer, compute=None):
    return _check(lib().moe_pool_retire(pool, layer, _s(compute)))


def moe_pool_stats(pool):
    st = PoolStats()
    _check(lib().moe_pool_stats(pool, C.byref(st)))
    return st


def moe_pool_access_counts(pool, layers, experts):
    """Per-(layer, expert) (hits, misses) since creation or the last reset, as
    two int64 numpy arrays of shape (layers, experts)."""
    import numpy as np
    h = np.zeros((layers, experts), np.int64)
    m = np.zeros((layers, experts), np.int64)
    _check(lib().moe_pool_access_counts(pool, h.ctypes.data, m.ctypes.data))
    return h, m


def moe_pool_reset(pool):
    return _check(lib().moe_pool_reset(pool))


def moe_pool_destroy(pool):
    return _check(lib().moe_pool_destroy(pool))
