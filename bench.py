#!/usr/bin/env python3
"""Benchmark of the W4A16 MoE hot path on one MI355X.

Default workload (decode): 16 stacked OLMoE-shaped MoE layers (hidden 2048,
64 experts, top-8, SwiGLU intermediate 1024, INT4 group 128 with fp16
scales, all experts resident in HBM), one token per step, fresh x0 ~ N(0,1)
per step, x_{l+1} = fp16(x_l + MoE_l(x_l)).  A step is route -> permute ->
routed expert FFN -> combine for all 16 layers.  Prints one JSON line.

    python bench.py [--steps 128] [--warmup 16] [--graph/--no-graph]
                    [--no-cpu-baseline] [--workload decode|batched|e512|qwen|partial|copy] [--T ...]

Other workloads (one JSON line each, not the headline):
  batched  single OLMoE-shaped layers at T = 64, 512, 4096 (grouped INT4
           FP16-MFMA path): per-call times, MFMA and HBM fractions.
  e512     single 512-expert layers (top-10, I = 512, FP16 shared expert with
           I_s = 512, Zipf(1.1) router bias) at T = 1, 256, 4096.
  qwen     single 60-expert layers (top-4, I = 1408, FP16 shared expert with
           I_s = 5632 scaled by a per-token sigmoid gate) at T = 1, 256, 4096.
  partial  16 layers with 30 of 64 experts per layer in an HBM slot pool and
           the INT4 source in pinned host memory: tokens/s and H2D GiB.
  copy     a 1 GiB device copy, the reference for HBM byte counters.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense FP16 MFMA, TFLOP/s


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


REGIMES = {"auto": 0, "decode": 1, "batched": 2, "small": 3}   # MOE_REGIME_* values
FMTS = {"sym": 0, "zp": 1}                                      # MOE_FMT_* values


def build_layers(cfg, layers, dev, torch, M, fmt=0):
    """Device-resident layers: weights drawn by moe_inputs (numpy), quantised
    and prepacked by the library's kernels (fmt: MOE_FMT_SYM or MOE_FMT_ZP)."""
    import moe_inputs as MI
    from int4_weight_only_router_amd.layer import MoELayer, blob_table
    _, total = M.moe_blob_layout_fmt(cfg.H, cfg.I, cfg.g, fmt)
    out = []
    for l in range(layers):
        t0 = time.time()
        blobs = torch.empty((cfg.E, total), dtype=torch.uint8, device=dev)
        for b0 in range(0, cfg.E, 32):
            ids = list(range(b0, min(cfg.E, b0 + 32)))
            n = len(ids)
            wg = torch.empty((n, cfg.I, cfg.H), dtype=torch.float32, device=dev)
            wu = torch.empty((n, cfg.I, cfg.H), dtype=torch.float32, device=dev)
            wd = torch.empty((n, cfg.H, cfg.I), dtype=torch.float32, device=dev)
            for i, (e, (g_, u_, d_)) in enumerate(MI.gen_experts(cfg, l, ids)):
                wg[i].copy_(torch.from_numpy(g_))
                wu[i].copy_(torch.from_numpy(u_))
                wd[i].copy_(torch.from_numpy(d_))
            canon = torch.empty((n, total), dtype=torch.uint8, device=dev)
            M.moe_quantize_experts_fmt(wg, wu, wd, n, cfg.H, cfg.I, cfg.g, fmt, canon)
            M.moe_prepack_experts_fmt(canon, n, cfg.H, cfg.I, cfg.g, fmt, blobs[b0:b0 + n])
            del wg, wu, wd, canon
        router = torch.from_numpy(MI.gen_router(cfg, l)).to(dev)
        b = MI.zipf_bias(cfg, l)
        bias = None if b is None else torch.from_numpy(b).to(dev)
        lay = MoELayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.g, router, blob_table(blobs), bias,
                       device=dev, fmt=fmt)
        lay._blobs = blobs
        out.append(lay)
        torch.cuda.synchronize()
        log("layer %d ready (%.1fs)" % (l, time.time() - t0))
    return out, total


# ------------------------------------------------------------- CPU baseline

def host_cpu():
    """CPU model, physical cores (distinct (package, core) pairs in
    /proc/cpuinfo, i.e. cores per socket x sockets) and the threads this
    process may use (affinity mask, OMP_NUM_THREADS).  Read from files; no
    tool is started."""
    model, cores = "unknown", set()
    try:
        phys = core = None
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            k, v = k.strip(), v.strip()
            if k == "model name" and model == "unknown":
                model = v
            elif k == "physical id":
                phys = v
            elif k == "core id":
                core = v
            elif not k and phys is not None:
                cores.add((phys, core))
                phys = core = None
        if phys is not None:
            cores.add((phys, core))
    except OSError:
        pass
    physical = len(cores) or os.cpu_count() or 1
    allowed = len(os.sched_getaffinity(0))
    omp = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(physical, allowed, omp) if omp > 0 else min(physical, allowed)
    return {"model": model, "physical_cores": physical, "allowed_cpus": allowed,
            "omp_num_threads": omp or None, "threads": max(1, threads)}


def cpu_baseline_decode(cfg, layers, steps, threads=1):
    """The oracle (plain C) on `steps` decode steps of the same 16-layer chain
    with `threads` worker threads (its rows spread over them; one token has
    k = 8 rows per layer, so at most 8 are busy); weight generation and
    oracle packing of the routed experts happen outside the timer."""
    import numpy as np
    import moe_inputs as MI
    import oracle as O
    O.set_threads(threads)
    routers = [MI.gen_router(cfg, l) for l in range(layers)]
    cache = {}
    busy = 0.0
    try:
        for s in range(steps):
            x = MI.gen_x(cfg, 1, step=s)
            for l in range(layers):
                t0 = time.perf_counter()
                idx, w, _ = O.route(x, routers[l], None, cfg.k)
                counts, offsets, perm, inv = O.permute(idx, cfg.E)
                busy += time.perf_counter() - t0
                need = [e for e in np.unique(idx) if (l, int(e)) not in cache]
                for e, wts in MI.gen_experts(cfg, l, need):
                    cache[(l, int(e))] = O.pack_expert(*wts, cfg.g)
                blobs = [cache.get((l, e)) for e in range(cfg.E)]
                t0 = time.perf_counter()
                y = O.expert_ffn(x, perm, offsets, blobs, cfg.H, cfg.I, cfg.E, cfg.k, cfg.g)
                out, _ = O.combine(y, inv, w, None, x)
                busy += time.perf_counter() - t0
                x = out
    finally:
        O.set_threads(0)
    return steps / busy, busy


# ------------------------------------------------------------------ decode

def _graph_time(torch, fn, reps):
    """Average duration of one call of fn (a sequence of launches on the
    current stream), captured once in a graph and replayed `reps` times
    between two events: launches run back to back, as in the timed loop."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


DECODE_KERNEL_SOURCES = ("int4_weight_only_router_amd/csrc/k_ffn_decode.hip",
                         "int4_weight_only_router_amd/csrc/k_decode_frag.h",
                         "int4_weight_only_router_amd/csrc/k_sort_common.h",
                         "int4_weight_only_router_amd/csrc/moe_common.h")


def sources_sha256(paths):
    """sha256 over the concatenated bytes of the files a kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()


def _profile_record(kernel_srcs, key):
    """The rocprofv3 figures recorded under profiles/traffic.json for a kernel
    (counter HBM bytes per launch, kernel-trace average duration), if the
    kernel's sources have not changed since they were taken (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[key]
        if sources_sha256(kernel_srcs) != rec["source_sha256"]:
            return None
        return rec
    except (OSError, KeyError, ValueError):
        return None


def hardware(torch):
    p = torch.cuda.get_device_properties(0)
    hw = {"gpu": p.name or "MI355X (gfx950)", "arch": getattr(p, "gcnArchName", None),
          "compute_units": p.multi_processor_count,
          "hbm_GiB": round(p.total_memory / 2 ** 30, 1),
          "rocm_hip": torch.version.hip, "torch": torch.__version__}
    # shader clock levels from sysfs (the level marked '*' is the current one);
    # read as a file, no tool is started
    hw["sclk"] = None
    try:
        import glob
        for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            levels = [l.strip() for l in open(f) if l.strip()]
            if levels:
                cur = [l for l in levels if l.endswith("*")]
                hw["sclk"] = {"current": cur[0] if cur else None, "levels": levels}
                break
    except OSError:
        pass
    return hw


def run_decode(args, torch, M):
    import numpy as np
    import moe_inputs as MI
    cfg = MI.OLMOE_DECODE
    dev = "cuda:0"
    L = cfg.layers
    fmt = FMTS[getattr(args, "fmt", "sym")]
    lays, blob_bytes = build_layers(cfg, L, dev, torch, M, fmt)
    K, W = args.steps, args.warmup
    xs = torch.from_numpy(np.concatenate([MI.gen_x(cfg, 1, step=s) for s in range(K + W)])).to(dev)
    bufs = [lay.buffers(1) for lay in lays]
    assert bufs[0].regime & ~(M.MOE_Y_TOKEN_ORDER | M.MOE_Y_PARTIAL_ORDER
                              | M.MOE_W4_ZERO_POINT) == M.MOE_REGIME_DECODE
    act = [torch.empty((1, cfg.H), dtype=torch.float16, device=dev) for _ in range(2)]

    fuse = not getattr(args, "no_fuse", False)
    split = fuse and not getattr(args, "route_in_combine", False)
    parts = torch.empty(M.moe_logit_partials_bytes() // 4, dtype=torch.float32, device=dev)

    def step_from(x):
        # with fuse, layer l's combine and layer l+1's route + permute are
        # one launch (moe_combine_route_permute); with split (the default),
        # layer l's combine hands on only layer l+1's logit partials and
        # layer l+1's expert launch routes from them
        # (moe_combine_route_partials + moe_expert_ffn_w4a16_routed), and
        # layer 0's from the partials of its input (moe_logit_partials);
        # the same bits in every form
        routed = False
        for l, lay in enumerate(lays):
            out = act[l & 1]
            if l == 0 and split:
                lay.logit_partials(x, parts)
                routed = True
            elif l == 0 or not fuse:
                lay.route_permute(x, bufs[l])
            if routed:
                lay.experts_routed(x, bufs[l], parts)
            else:
                lay.experts(x, bufs[l])
            routed = False
            if fuse and l + 1 < L:
                if split:
                    lay.combine_partials_next(bufs[l], lays[l + 1], parts, residual=x, out=out)
                    routed = True
                else:
                    lay.combine_route_next(bufs[l], lays[l + 1], bufs[l + 1], residual=x,
                                           out=out)
            else:
                lay.combine(bufs[l], residual=x, out=out)
            x = out
        return x

    log("warmup %d steps" % W)
    for s in range(W):
        step_from(xs[s:s + 1])
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        # one captured step: gather this step's token into a fixed buffer,
        # run the 16 layers on it, advance the token index (all on the GPU,
        # so a step is one replay)
        xin = torch.empty((1, cfg.H), dtype=torch.float16, device=dev)
        sel = torch.zeros(1, dtype=torch.int64, device=dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            torch.index_select(xs, 0, sel, out=xin)
            step_from(xin)
            sel.add_(1)
        graph = (g, sel)
        for s in range(3):
            sel.fill_(s % (K + W))   # every replay reads a row of xs
            g.replay()
        torch.cuda.synchronize()

    log("timed %d steps (graph=%s)" % (K, bool(graph)))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph:
        g, sel = graph
        sel.fill_(W)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(W, W + K):
            g.replay()
    else:
        for s in range(W, W + K):
            step_from(xs[s:s + 1])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # per-kernel launch durations (HIP events on the launch stream): each
    # layer's kernel once per replay, all 16 layers in turn (415 MB of
    # expert weights per pass, more than the 256 MB Infinity Cache)
    reps = max(4, K // 8)
    x0 = xs[0:1]
    t_route = _graph_time(torch, lambda: [lay.route_permute(x0, bufs[l])
                                          for l, lay in enumerate(lays)], reps) / L
    t_ffn = _graph_time(torch, lambda: [lay.experts(x0, bufs[l])
                                        for l, lay in enumerate(lays)], reps) / L
    t_comb = _graph_time(torch, lambda: [lay.combine(bufs[l], residual=x0, out=act[0])
                                         for l, lay in enumerate(lays)], reps) / L
    touched = [int((b.counts.cpu().numpy() > 0).sum()) for b in bufs]
    t_cr = _graph_time(torch, lambda: [lays[l].combine_route_next(bufs[l], lays[l + 1],
                                                                  bufs[l + 1], residual=x0,
                                                                  out=act[0])
                                       for l in range(L - 1)], reps) / (L - 1)
    t_cp = _graph_time(torch, lambda: [lays[l].combine_partials_next(bufs[l], lays[l + 1], parts,
                                                                     residual=x0, out=act[0])
                                       for l in range(L - 1)], reps) / (L - 1)
    t_ffn_r = _graph_time(torch, lambda: [lays[l].experts_routed(x0, bufs[l], parts)
                                          for l in range(1, L)], reps) / (L - 1)
    t_lp = _graph_time(torch, lambda: [lay.logit_partials(x0, parts) for lay in lays], reps) / L
    ffn_bytes = int(np.mean(touched)) * blob_bytes + cfg.H * 2   # INT4 + scales of routed experts, x
    # the decode kernel as the step runs it: with split, layers 1..15 route
    # inside it from the logit partials
    t_dom = t_ffn_r if split else t_ffn
    achieved = ffn_bytes / (t_dom * 1e-3) / 1e9
    ms_step = elapsed * 1e3 / K
    prof = _profile_record(DECODE_KERNEL_SOURCES, "ffn_decode_kernel olmoe_decode") or {}
    traffic = prof.get("hbm_bytes_per_launch")
    trace_us = prof.get("trace_avg_us")
    res = {
        "metric": "MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA util (batched), W4A16",
        "value": round(K / elapsed, 2),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int4-weights/f16-activations/f32-accumulate" if fmt == 0 else
                 "int4-zero-point-weights/f16-activations/f32-accumulate",
        "data": "synthetic (seeded numpy draws: x ~ N(0,1), router ~ N(0,0.02), experts "
                "~ N(0,0.02) quantised INT4 g128%s)" % ("" if fmt == 0 else ", zero point per group"),
        "config": {"workload": "olmoe_decode: 16 MoE layers H=2048 E=64 top-8 I=1024 g=128, "
                               "1 token/step, all experts resident",
                   "layers": L, "tokens_per_step": 1, "graph": bool(graph),
                   "format": "sym" if fmt == 0 else "zp", "combine_route_fused": fuse,
                   "route_in_ffn": split},
        "layer_tokens_per_s": round(K * L / elapsed, 1),
        "per_layer_us": {"route+permute": round(t_route * 1e3, 2),
                         "expert_ffn": round(t_ffn * 1e3, 2),
                         "combine": round(t_comb * 1e3, 2),
                         "combine+next_route": round(t_cr * 1e3, 2),
                         "combine+next_logit_partials": round(t_cp * 1e3, 2),
                         "route_from_partials+expert_ffn": round(t_ffn_r * 1e3, 2),
                         "first_layer_logit_partials": round(t_lp * 1e3, 2)},
        "roofline": {"kernel": "ffn_decode_kernel (%s, DECODE)" % (
                         "moe_expert_ffn_w4a16_routed" if split else "moe_expert_ffn_w4a16"),
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "alg_bytes_per_launch": ffn_bytes,
                     "avg_launch_us": round(t_dom * 1e3, 3),
                     "timing": "HIP events around a graph of the kernel's 16 layer launches "
                               "on its launch stream, averaged per launch",
                     # the same kernel's average duration in the committed
                     # rocprofv3 kernel trace (null once the sources changed)
                     "trace_avg_launch_us": trace_us,
                     "frac_trace": None if not trace_us else
                     round(ffn_bytes / (trace_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    res["hardware"] = hardware(torch)
    if args.extras:
        log("batched leg: one OLMoE-shaped layer at 4096 tokens")
        res["batched_olmoe_t4096"] = batched_leg(torch, M)
        torch.cuda.empty_cache()
        log("partial-residency leg")
        res["partial_residency"] = partial_leg(torch, M)
    if args.cpu_baseline:
        cpu = host_cpu()
        log("cpu baseline (oracle, 1 thread)")
        sps1, busy1 = cpu_baseline_decode(cfg, L, args.cpu_steps, 1)
        nt = cpu["threads"]
        log("cpu baseline (oracle, %d threads)" % nt)
        spsn, busyn = cpu_baseline_decode(cfg, L, args.cpu_steps_mt, nt)
        used = min(nt, cfg.k)   # one token: k rows per layer to spread
        res["cpu_baseline"] = {
            "value": round(spsn, 4), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": "%d decode steps x 16 layers (route, permute, fp64 expert FFN, combine) "
                      "with %d OpenMP threads, %d of them busy (k = 8 rows per layer); "
                      "%.1f s of CPU work" % (args.cpu_steps_mt, nt, used, busyn),
            "cpu_model": cpu["model"], "physical_cores": cpu["physical_cores"],
            "allowed_cpus": cpu["allowed_cpus"], "threads": nt,
            "single_thread": {"value": round(sps1, 4), "unit": "tokens/s", "cores": 1,
                              "sample": "%d decode steps x 16 layers, %.1f s of CPU work"
                                        % (args.cpu_steps, busy1)}}
    return res


# ----------------------------------------------------------------- batched

def run_batched(args, torch, M, cfg):
    """Single layers of `cfg` at each batch size.  Each part of the layer
    (route+permute, routed expert FFN, shared expert, combine) and the whole
    layer is captured in a graph over NC >= 16 copies of the layer's weights at
    distinct addresses (NC x layer bytes > 3x the 256 MB last-level cache, so
    no copy is still cached when its turn comes) and replayed; the average
    per call is reported.  With it: the MFMA fraction of the routed FFN
    (routed FLOPs), its HBM fraction (touched expert blobs only: the bound at
    small T) and the HBM fraction of the whole layer (algorithmic bytes:
    touched expert blobs, router, shared weights, x, out)."""
    import numpy as np
    import moe_inputs as MI
    from int4_weight_only_router_amd.layer import MoELayer, blob_table
    dev = "cuda:0"
    lays, blob_bytes = build_layers(cfg, 1, dev, torch, M, FMTS[getattr(args, "fmt", "sym")])
    base = lays[0]
    shared = gate = None
    if cfg.Is:
        shared = tuple(torch.from_numpy(w).to(dev) for w in MI.gen_shared(cfg))
        if cfg.shared_gate:
            gate = torch.from_numpy(MI.gen_shared_gate(cfg)).to(dev)
    # at least 16 calls per captured graph, so that the replay's own launch
    # cost is shared (and the touched weights of 16 small-T calls still
    # exceed the last-level cache); every copy has its own shared weights too
    nc = max(16, -(-3 * 256 * 2 ** 20 // (cfg.E * blob_bytes)))
    # shared expert on a side stream when its weights are large (60-expert
    # layer: 69 MB); with the 512-expert layer's 6 MB it only delays routing
    overlap = bool(cfg.Is) and 3 * cfg.H * cfg.Is * 2 >= 32 * 2 ** 20
    copies = [base]
    for _ in range(nc - 1):
        bl = base._blobs.clone()
        sh = None if shared is None else tuple(w.clone() for w in shared)
        lay = MoELayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.g, base.router, blob_table(bl), base.bias,
                       sh, device=dev, shared_gate=gate, overlap_shared=overlap, fmt=base.fmt)
        lay._blobs = bl
        copies.append(lay)
    base.shared, base.shared_gate, base.overlap_shared = shared, gate, overlap
    Ts = [int(t) for t in args.T.split(",")] if args.T else list(cfg.T)
    reps = max(1, args.steps // nc)
    lines = []
    for T in Ts:
        x = torch.from_numpy(MI.gen_x(cfg, T)).to(dev)
        bufs = [lay.buffers(T, REGIMES[args.regime]) for lay in copies]
        for _ in range(max(1, args.warmup)):
            for lay, b in zip(copies, bufs):
                lay.forward(x, b)
        torch.cuda.synchronize()

        def each(fn):
            return lambda: [fn(lay, b) for lay, b in zip(copies, bufs)]

        def ffn(lay, b):
            M.moe_expert_ffn_w4a16(x, b.perm, b.offsets, lay.table, T, cfg.H, cfg.I, cfg.E,
                                   cfg.k, cfg.g, b.regime, b.y, b.y_dtype, b.y_slices, b.ffn_ws,
                                   0 if b.ffn_ws is None else b.ffn_ws.numel())

        def shr(lay, b):
            wg, wu, wd = lay.shared
            M.moe_shared_ffn_f16(x, wg, wu, wd, T, cfg.H, cfg.Is, b.shared_out, b.shared_ws,
                                 b.shared_ws.numel())

        parts = {"route_permute": each(lambda lay, b: lay.route_permute(x, b)),
                 "expert_ffn": each(ffn), "combine": each(lambda lay, b: lay.combine(b, x=x)),
                 "layer": each(lambda lay, b: lay.forward(x, b))}
        if shared is not None:
            parts["shared"] = each(shr)
        us = {k: _graph_time(torch, fn, reps) * 1e3 / nc for k, fn in parts.items()}
        b = bufs[0]
        counts = b.counts.cpu().numpy()
        touched = int((counts > 0).sum())
        f_routed = 2.0 * T * cfg.k * 3 * cfg.H * cfg.I
        f_shared = 2.0 * T * 3 * cfg.H * cfg.Is
        f_router = 2.0 * T * cfg.E * cfg.H
        b_alg = (touched * blob_bytes + cfg.E * cfg.H * 2 + 3 * cfg.H * cfg.Is * 2
                 + 2 * T * cfg.H * 2 + (cfg.H * 2 if cfg.shared_gate else 0))
        tf = f_routed / (us["expert_ffn"] * 1e-6) / 1e12
        ffn_bytes = touched * blob_bytes
        reg = b.regime & ~(M.MOE_Y_TOKEN_ORDER | M.MOE_Y_PARTIAL_ORDER | M.MOE_W4_ZERO_POINT)
        line = {"T": T, "regime": {1: "decode", 2: "batched", 3: "small"}.get(reg, reg),
                "experts_touched": touched, "max_rows_per_expert": int(counts.max()),
                "us": {k: round(v, 1) for k, v in us.items()},
                "expert_ffn_alg_GB": round(ffn_bytes / 1e9, 4),
                "expert_ffn_hbm_frac": round(ffn_bytes / (us["expert_ffn"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "routed_tflops": round(tf, 1), "routed_mfma_frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                "layer_tflops": round((f_routed + f_shared + f_router) / (us["layer"] * 1e-6) / 1e12, 1),
                "layer_alg_GB": round(b_alg / 1e9, 4),
                "layer_hbm_frac": round(b_alg / (us["layer"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        if cfg.Is:
            line["shared_tflops"] = round(f_shared / (us["shared"] * 1e-6) / 1e12, 1)
            line["shared_hbm_frac"] = round(3 * cfg.H * cfg.Is * 2 / (us["shared"] * 1e-6) / 1e9
                                            / HBM_PEAK_GBS, 4)
        lines.append(line)
        log(str(line))
    return {"workload": cfg.name, "weight_copies": nc, "regime": args.regime,
            "format": getattr(args, "fmt", "sym"),
            "config": {"H": cfg.H, "E": cfg.E, "k": cfg.k, "I": cfg.I, "g": cfg.g, "Is": cfg.Is,
                       "shared_gate": cfg.shared_gate, "zipf_s": cfg.zipf_s,
                       "shared_on_side_stream": overlap},
            "results": lines}


def run_partial(args, torch, M):
    """Partial residency: 16 OLMoE-shaped layers, C of 64 experts per layer
    resident in HBM slots (+ S spares), the full INT4 source in pinned host
    memory; per token and layer one moe_pool_layer_forward call: route (GPU)
    -> routed ids to the host -> prepare (misses copied H2D on a side stream)
    -> expert FFN through the published table -> retire -> combine.
    Protocol: `blocks`
    fresh pools, each a 64-token warmup then `prompts` x `tokens` tokens.
    --policy pinned: a profile pass first (`profile_prompts` other prompts of
    the same workload, through the decayed-counter pool) counts the routed
    experts per layer; every block then pins each layer's C most counted
    experts (moe_pool_pin).  Either way the report carries the static hit
    ceiling of the measured trace: the C most routed experts of each layer in
    hindsight, the most any fixed set can hit."""
    import numpy as np
    import moe_inputs as MI
    cfg = MI.PARTIAL
    dev = "cuda:0"
    L = cfg.layers
    lays, blob_bytes = build_layers(cfg, L, dev, torch, M)
    src = torch.empty((L, cfg.E, blob_bytes), dtype=torch.uint8, pin_memory=True)
    for l, lay in enumerate(lays):
        src[l].copy_(lay._blobs)
        lay._blobs = None
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    # pinned -> HBM rate of one expert blob copy (the miss path's unit), median
    # of 16 copies timed with events on a side stream
    tmp = torch.empty(blob_bytes, dtype=torch.uint8, device=dev)
    cs = torch.cuda.Stream()
    cms = []
    with torch.cuda.stream(cs):
        for e in range(17):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cs)
            tmp.copy_(src[e % L, e % cfg.E], non_blocking=True)
            e1.record(cs)
            e1.synchronize()
            if e:
                cms.append(e0.elapsed_time(e1))
    del tmp
    cms.sort()
    h2d_gbs = blob_bytes / (cms[len(cms) // 2] * 1e-3) / 1e9
    ptrs = [src[l, e].data_ptr() for l in range(L) for e in range(cfg.E)]
    pc = M.PoolConfig(layers=L, experts=cfg.E, topk=cfg.k, capacity=cfg.capacity,
                      spares=cfg.spares, decay_shift=args.decay_shift, expert_bytes=blob_bytes)
    pool = M.moe_pool_create(pc, ptrs)
    bufs = [lay.buffers(1) for lay in lays]
    act = [torch.empty((1, cfg.H), dtype=torch.float16, device=dev) for _ in range(2)]
    host_ids = torch.empty(cfg.k, dtype=torch.int32, pin_memory=True)
    largs = [lay.pool_args(b, host_ids) for lay, b in zip(lays, bufs)]
    stream = torch.cuda.current_stream()
    step = M.PoolStats()
    trace_layers, trace_ids = [], []
    pinned = None
    # access map of the measured tokens: per-(layer, expert) hits and misses
    # (the pool's own counters) and a hit/miss log per (token, layer)
    acc_hits = np.zeros((L, cfg.E), np.int64)
    acc_misses = np.zeros((L, cfg.E), np.int64)
    hm_log = []

    def token(x0, record, log_hm=False):
        # one native call per layer: route, ids to the host, prepare (misses
        # copied), expert FFN through the published table, retire, combine
        x = x0.data_ptr()
        misses = 0
        row = []
        for l in range(L):
            a = largs[l]
            out = act[l & 1].data_ptr()
            a.x_f16, a.residual_f16, a.out_f16 = x, x, out
            M.moe_pool_layer_forward(pool, l, a, stream, step)
            misses += step.misses
            if log_hm:
                row.append((step.hits, step.misses))
            if record:
                trace_layers.append(l)
                trace_ids.append(host_ids.numpy().copy())
            x = out
        if log_hm:
            hm_log.append(row)
        return misses

    blocks = []
    try:
        if args.policy == "pinned":
            # profile pass: prompts of their own (ids past the measured ones)
            M.moe_pool_reset(pool)
            for p in range(args.profile_prompts):
                for i in range(args.tokens):
                    token(torch.from_numpy(MI.gen_prompt_token(cfg, 1000 + p, i)).to(dev), True)
            torch.cuda.synchronize()
            counts = np.zeros((L, cfg.E), np.int64)
            for l, ids in zip(trace_layers, trace_ids):
                counts[l, ids] += 1
            trace_layers.clear()
            trace_ids.clear()
            # the C most counted experts per layer, ties to the lower id
            pinned = np.sort(np.argsort(-counts, axis=1, kind="stable")[:, :cfg.capacity], axis=1)
            log("profile: %d tokens" % (args.profile_prompts * args.tokens))
        for blk in range(args.blocks):
            M.moe_pool_reset(pool)
            if pinned is not None:
                for l in range(L):
                    M.moe_pool_pin(pool, l, pinned[l])
            for i in range(cfg.warmup_tokens):
                token(torch.from_numpy(MI.gen_prompt_token(cfg, -1, i)).to(dev), blk == 0)
            torch.cuda.synchronize()
            base = M.moe_pool_stats(pool)
            h0, m0 = M.moe_pool_access_counts(pool, L, cfg.E)
            x0s = [[torch.from_numpy(MI.gen_prompt_token(cfg, p, i)).to(dev)
                    for i in range(args.tokens)] for p in range(args.prompts)]
            busy = 0.0
            ntok = 0
            for p in range(args.prompts):
                token(x0s[p][0], blk == 0, True)      # first token: outside the rate
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for i in range(1, args.tokens):
                    token(x0s[p][i], blk == 0, True)
                torch.cuda.synchronize()
                busy += time.perf_counter() - t0
                ntok += args.tokens - 1
            st = M.moe_pool_stats(pool)
            h1, m1 = M.moe_pool_access_counts(pool, L, cfg.E)
            acc_hits += h1 - h0
            acc_misses += m1 - m0
            blocks.append({"tokens_per_s": ntok / busy,
                           "h2d_bytes": st.h2d_bytes - base.h2d_bytes,
                           "hits": st.hits - base.hits, "misses": st.misses - base.misses})
            log("block %d: %.1f tokens/s, %.2f GiB H2D" % (
                blk, blocks[-1]["tokens_per_s"], blocks[-1]["h2d_bytes"] / 2 ** 30))
    finally:
        M.moe_pool_destroy(pool)
    tl = np.array(trace_layers, np.int32)
    ti = np.array(trace_ids, np.int32)
    nw = cfg.warmup_tokens * L
    # static ceiling of block 0's measured trace: per layer the C experts
    # routed most often in hindsight
    mc = np.zeros((L, cfg.E), np.int64)
    for l, ids in zip(tl[nw:], ti[nw:]):
        mc[l, ids] += 1
    ceiling = float(np.sort(mc, axis=1)[:, ::-1][:, :cfg.capacity].sum() / max(1, mc.sum()))
    rates = [b["tokens_per_s"] for b in blocks]
    tot_tok = args.blocks * args.prompts * (args.tokens - 1)
    tot_time = sum(args.prompts * (args.tokens - 1) / r for r in rates)
    h2d = sum(b["h2d_bytes"] for b in blocks)
    hits = sum(b["hits"] for b in blocks)
    misses = sum(b["misses"] for b in blocks)
    # the local-inference explainer's step-5 model of a token's time:
    # t_token = t_calc + bytes outside HBM / link bandwidth.  t_calc is the
    # HBM roofline of the resident work (per layer: k routed blobs, router,
    # x/out/residual); bytes outside = misses per token x blob bytes
    mpt = misses / max(1, args.blocks * args.prompts * args.tokens)
    t_calc = L * (cfg.k * blob_bytes + cfg.E * cfg.H * 2 + 3 * cfg.H * 2) / (HBM_PEAK_GBS * 1e9)
    t_meas = tot_time / tot_tok
    bound = {"t_calc_ms": round(t_calc * 1e3, 4),
             "h2d_GBs_measured_one_blob": round(h2d_gbs, 1),
             "t_token_bound_ms": round((t_calc + mpt * blob_bytes / (h2d_gbs * 1e9)) * 1e3, 4),
             "t_token_measured_ms": round(t_meas * 1e3, 4),
             "frac": round((t_calc + mpt * blob_bytes / (h2d_gbs * 1e9)) / t_meas, 4),
             "t_token_bound_pcie5_ms": round((t_calc + mpt * blob_bytes / 64e9) * 1e3, 4),
             "frac_pcie5": round((t_calc + mpt * blob_bytes / 64e9) / t_meas, 4)}
    access = access_summary(acc_hits, acc_misses, cfg.capacity, hm_log)
    if args.access_out:
        with open(args.access_out, "w") as f:
            json.dump({"layers": L, "experts": cfg.E, "capacity": cfg.capacity,
                       "policy": args.policy, "hits": acc_hits.tolist(),
                       "misses": acc_misses.tolist(),
                       "hit_miss_log": [[list(hm) for hm in row] for row in hm_log]}, f)
        access["file"] = args.access_out
    return {
        "workload": "olmoe_partial: 16 layers, %d of 64 experts resident + %d spares per layer, "
                    "Zipf(1.0) router bias, %d blocks x (64 warmup + %d prompts x %d tokens)"
                    % (cfg.capacity, cfg.spares, args.blocks, args.prompts, args.tokens),
        "decode_tokens_per_s_pooled": round(tot_tok / tot_time, 2),
        "block_tokens_per_s": [round(r, 2) for r in rates],
        "block_spread": round((max(rates) - min(rates)) / max(rates), 4),
        "h2d_GiB_measured": round(h2d / 2 ** 30, 3),
        "hit_rate": round(hits / max(1, hits + misses), 4),
        "misses_per_token": round(misses / (args.blocks * args.prompts * args.tokens), 3),
        "hit_ceiling_static_block0": round(ceiling, 4),
        "pool_misses_block0": blocks[0]["misses"],
        "policy": args.policy,
        "decay_shift": args.decay_shift if pinned is None else None,
        "profile_tokens": args.profile_prompts * args.tokens if pinned is not None else 0,
        "t_token_model": bound,
        "access": access,
    }


def access_summary(hits, misses, C, hm_log):
    """A few figures of the per-(layer, expert) access map of the measured
    tokens (all blocks): how many experts each layer touched, the share of a
    layer's uses taken by its C most used experts (the static hit ceiling of
    the whole run), how concentrated the misses are, the hottest (layer,
    expert) pairs, and from the per-(token, layer) log the share of layer
    calls that missed at all."""
    import numpy as np
    uses = hits + misses
    tot = max(1, int(uses.sum()))
    per_layer = np.maximum(1, uses.sum(axis=1))
    topc = np.sort(uses, axis=1)[:, ::-1][:, :C].sum(axis=1) / per_layer
    ms = np.sort(misses, axis=1)[:, ::-1]
    miss8 = ms[:, :8].sum() / max(1, int(misses.sum()))
    flat = np.argsort(-uses, axis=None, kind="stable")[:5]
    hottest = [[int(i // uses.shape[1]), int(i % uses.shape[1]),
                int(uses.flat[i]), int(misses.flat[i])] for i in flat]
    calls = [hm for row in hm_log for hm in row]
    missed_calls = sum(1 for h, m in calls if m > 0)
    return {"uses": tot,
            "touched_per_layer": [int(v) for v in (uses > 0).sum(axis=1)],
            "top_C_use_share_per_layer": [round(float(v), 4) for v in topc],
            "miss_share_8_most_missed_per_layer": round(float(miss8), 4),
            "hottest_layer_expert_uses_misses": hottest,
            "layer_calls": len(calls),
            "layer_calls_with_a_miss": round(missed_calls / max(1, len(calls)), 4)}


def batched_leg(torch, M, T=4096):
    """The batched OLMoE-shaped layer at T tokens (grouped INT4 -> FP16 MFMA
    path), timed as `--workload batched` does: routed-FFN MFMA fraction on
    the routed FLOPs and the whole layer's time."""
    import moe_inputs as MI
    a = argparse.Namespace(T=str(T), regime="auto", steps=64, warmup=2)
    r = run_batched(a, torch, M, MI.OLMOE_BATCHED)
    line = r["results"][0]
    return {"workload": "olmoe_batched: one layer H=2048 E=64 top-8 I=1024 g=128, T=%d" % T,
            "regime": line["regime"], "us": line["us"],
            "routed_tflops": line["routed_tflops"], "routed_mfma_frac": line["routed_mfma_frac"],
            "mfma_peak_tflops": MFMA_F16_PEAK_TFLOPS,
            "layer_tokens_per_s": round(T / (line["us"]["layer"] * 1e-6), 1),
            "weight_copies": r["weight_copies"]}


def partial_leg(torch, M, prompts=2, tokens=64):
    """A short partial-residency run (one block: 64 warmup tokens, then
    `prompts` x `tokens` tokens) with the explainer's t_token bound."""
    a = argparse.Namespace(blocks=1, prompts=prompts, tokens=tokens, decay_shift=3,
                           policy="decay", profile_prompts=0, access_out="")
    r = run_partial(a, torch, M)
    keep = ("workload", "decode_tokens_per_s_pooled", "h2d_GiB_measured", "hit_rate",
            "misses_per_token", "pool_misses_block0", "t_token_model")
    return {k: r[k] for k in keep}


def run_copy(args, torch, M):
    """A plain device-to-device copy of known size: the reference for scaling
    the HBM byte counters (FETCH_SIZE / WRITE_SIZE) of the other kernels."""
    nbytes = 1 << 30
    src = torch.empty(nbytes // 2, dtype=torch.float16, device="cuda:0").normal_()
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms = []
    for _ in range(args.steps):
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    ms.sort()
    med = ms[len(ms) // 2]
    return {"workload": "copy", "bytes_read_per_launch": nbytes, "bytes_written_per_launch": nbytes,
            "median_ms": round(med, 4), "GBs_read_plus_write": round(2 * nbytes / med / 1e6, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", choices=["decode", "batched", "e512", "qwen", "partial", "copy"],
                    default="decode")
    ap.add_argument("--T", default="", help="batched/e512/qwen: comma-separated batch sizes")
    ap.add_argument("--fmt", choices=["sym", "zp"], default="sym",
                    help="expert blob format: symmetric INT4, or INT4 with a zero point per "
                         "group (decode/batched/e512/qwen)")
    ap.add_argument("--regime", choices=sorted(REGIMES), default="auto",
                    help="batched/e512/qwen: routed-FFN regime (auto: the library's choice)")
    ap.add_argument("--blocks", type=int, default=3)
    ap.add_argument("--prompts", type=int, default=12)
    ap.add_argument("--tokens", type=int, default=128)
    ap.add_argument("--decay-shift", type=int, default=3)
    ap.add_argument("--policy", choices=["decay", "pinned"], default="decay",
                    help="partial: decayed-counter eviction, or a profile-pinned resident set")
    ap.add_argument("--access-out", default="",
                    help="partial: write the per-(layer, expert) access map and the "
                         "per-(token, layer) hit/miss log to this JSON file")
    ap.add_argument("--profile-prompts", type=int, default=4,
                    help="partial --policy pinned: prompts of the profile pass")
    ap.add_argument("--no-fuse", dest="no_fuse", action="store_true", default=False,
                    help="decode: separate combine and next-layer route launches")
    ap.add_argument("--route-in-combine", dest="route_in_combine", action="store_true",
                    default=False,
                    help="decode: route each next layer inside the fused combine launch "
                         "(moe_combine_route_permute) instead of inside its expert launch")
    ap.add_argument("--graph", dest="graph", action="store_true", default=True)
    ap.add_argument("--no-graph", dest="graph", action="store_false")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false", default=True)
    ap.add_argument("--cpu-steps", type=int, default=2,
                    help="decode steps of the one-thread oracle leg")
    ap.add_argument("--cpu-steps-mt", type=int, default=8,
                    help="decode steps of the multi-threaded oracle leg")
    ap.add_argument("--no-extras", dest="extras", action="store_false", default=True,
                    help="decode: skip the batched (4096 tokens) and partial-residency legs")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs the layer on one MI355X and "
              "has no multi-GPU path (expert-parallel sharding is described in the design "
              "notes, not implemented).", file=sys.stderr)
        sys.exit(2)
    import torch
    import int4_weight_only_router_amd as M
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    M.lib()
    if args.workload == "decode":
        res = run_decode(args, torch, M)
    elif args.workload in ("batched", "e512", "qwen"):
        import moe_inputs as MI
        res = run_batched(args, torch, M, {"batched": MI.OLMOE_BATCHED, "e512": MI.E512,
                                           "qwen": MI.QWEN}[args.workload])
    elif args.workload == "partial":
        res = run_partial(args, torch, M)
    else:
        res = run_copy(args, torch, M)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
