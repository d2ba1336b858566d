"""Helpers of the GPU tests: device layers built from the seeded inputs
(quantised and prepacked by the library's own kernels), oracle blobs built
from the same draws by the oracle's own quantiser, tolerance checks, and a
progress line on the real stderr before each GPU step."""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import int4_weight_only_router_amd as M
from int4_weight_only_router_amd.layer import MoELayer, blob_table
import moe_inputs as MI
import oracle as O

DEV = "cuda:0"
ATOL = 2e-2      # max |delta| on outputs
RTOL_L2 = 1e-2   # relative L2 on outputs
WTOL = 1e-5      # routing weights


def say(msg):
    sys.__stderr__.write("[gpu] %s\n" % msg)
    sys.__stderr__.flush()


def f16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def device_experts(cfg, layer, experts=None, batch=32, fmt=M.MOE_FMT_SYM):
    """Prepacked device blobs [E, bytes] of a layer; canonical blobs too."""
    experts = list(range(cfg.E)) if experts is None else list(experts)
    _, total = M.moe_blob_layout_fmt(cfg.H, cfg.I, cfg.g, fmt)
    dev = torch.empty((cfg.E, total), dtype=torch.uint8, device=DEV)
    canon = torch.empty((cfg.E, total), dtype=torch.uint8, device=DEV)
    for b0 in range(0, len(experts), batch):
        ids = experts[b0:b0 + batch]
        n = len(ids)
        wg = torch.empty((n, cfg.I, cfg.H), dtype=torch.float32, device=DEV)
        wu = torch.empty((n, cfg.I, cfg.H), dtype=torch.float32, device=DEV)
        wd = torch.empty((n, cfg.H, cfg.I), dtype=torch.float32, device=DEV)
        for i, (e, (g_, u_, d_)) in enumerate(MI.gen_experts(cfg, layer, ids)):
            wg[i].copy_(torch.from_numpy(g_))
            wu[i].copy_(torch.from_numpy(u_))
            wd[i].copy_(torch.from_numpy(d_))
        cb = torch.empty((n, total), dtype=torch.uint8, device=DEV)
        db = torch.empty((n, total), dtype=torch.uint8, device=DEV)
        M.moe_quantize_experts_fmt(wg, wu, wd, n, cfg.H, cfg.I, cfg.g, fmt, cb)
        M.moe_prepack_experts_fmt(cb, n, cfg.H, cfg.I, cfg.g, fmt, db)
        idx = torch.tensor(ids, device=DEV)
        dev[idx] = db
        canon[idx] = cb
        del wg, wu, wd
    torch.cuda.synchronize()
    return dev, canon


class OracleBlobs:
    """Lazily packed oracle blobs of one layer (same draws, oracle quantiser)."""

    def __init__(self, cfg, layer, fmt=O.FMT_SYM):
        self.cfg, self.layer, self.fmt, self.cache = cfg, layer, fmt, {}

    def get(self, experts):
        c = self.cfg
        need = [e for e in sorted(set(int(e) for e in experts)) if e not in self.cache]
        # draws and oracle packing in threads (numpy and the C oracle release
        # the GIL); every expert is still packed by the oracle's quantiser
        with ThreadPoolExecutor(8) as ex:
            packed = ex.map(lambda e: (e, O.pack_expert(*MI.gen_expert(c, self.layer, e), c.g,
                                                        self.fmt)), need)
            for e, blob in packed:
                self.cache[e] = blob
        return [self.cache.get(e) for e in range(c.E)]


_EXPERT_CACHE = {}


def cached_experts(cfg, layer, fmt=M.MOE_FMT_SYM):
    key = (cfg.cid, cfg.H, cfg.E, cfg.I, cfg.g, layer, fmt)
    if key not in _EXPERT_CACHE:
        if len(_EXPERT_CACHE) >= 3:
            _EXPERT_CACHE.pop(next(iter(_EXPERT_CACHE)))
        say("build experts cfg=%s layer=%d fmt=%d" % (cfg.name, layer, fmt))
        _EXPERT_CACHE[key] = device_experts(cfg, layer, fmt=fmt)[0]
    return _EXPERT_CACHE[key]


def make_layer(cfg, layer=0, shared=True, fmt=M.MOE_FMT_SYM):
    dev = cached_experts(cfg, layer, fmt)
    router = f16(MI.gen_router(cfg, layer))
    b = MI.zipf_bias(cfg, layer)
    bias = None if b is None else torch.from_numpy(b).to(DEV)
    sh = None
    if shared and cfg.Is:
        sh = tuple(f16(w) for w in MI.gen_shared(cfg))
    gate = f16(MI.gen_shared_gate(cfg)) if (sh is not None and cfg.shared_gate) else None
    lay = MoELayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.g, router, blob_table(dev), bias, sh,
                   device=DEV, shared_gate=gate, fmt=fmt)
    lay._blobs = dev            # keep the storage alive
    return lay


def check_close(got, ref, what, atol=ATOL, rtol_l2=RTOL_L2):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    d = np.abs(got - ref)
    mx = float(d.max()) if d.size else 0.0
    l2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    assert mx <= atol and l2 <= rtol_l2, "%s: max|d|=%.3g (<= %g), relL2=%.3g (<= %g)" % (
        what, mx, atol, l2, rtol_l2)
    return mx, l2


def sample_rows(offsets, n_per_expert=2, max_extra=64, seed=0):
    """Sorted rows to check: the first and last row of every non-empty expert
    bucket (tile edges: at most 2E rows, always all of them), plus up to
    `max_extra` seeded random rows from inside the buckets."""
    rng = np.random.default_rng(seed)
    edges, extra = set(), set()
    E = len(offsets) - 1
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            edges.add(a)
            edges.add(b - 1)
            for r in rng.integers(a, b, n_per_expert):
                extra.add(int(r))
    extra = sorted(extra - edges)
    if len(extra) > max_extra:
        extra = rng.choice(extra, max_extra, replace=False).tolist()
    return np.array(sorted(edges | set(extra)), np.int32)


def pm_positions(H):
    """Stored column of each column in the decode partials' partial-major
    order (the header's rule: column c of chunk u = 64 m + j, j < 64, goes to
    8 (j q + m) + c mod 8 with q = ceil(H / 8 / 64))."""
    q = (H // 8 + 63) // 64
    c = np.arange(H)
    u = c // 8
    return ((u % 64) * q + u // 64) * 8 + c % 8


def y_plain(b):
    """A layer's y as numpy, decode partial columns back in plain order."""
    y = b.y.detach().cpu().numpy()
    if b.y_dtype == M.MOE_DTYPE_F32_PM:
        y = y[..., pm_positions(y.shape[-1])]
    return y
