"""Seeded synthetic inputs for the W4A16 MoE layer.

This module only draws numbers: activations, router weights, full-precision
expert weights (before any quantisation), shared-expert weights, the per-layer
Zipf logit bias and the partial-residency token streams.  It holds none of the
layer's arithmetic (no quantiser, no routing, no FFN), so the CPU oracle under
``oracle/`` and the HIP library can both take their inputs from here without
sharing any method code.

Every tensor comes from its own numpy ``Generator`` seeded by
``SeedSequence(seed, spawn_key=(config, tensor, layer, expert, step))``, so any
single expert or token can be regenerated on its own (the oracle regenerates
only the experts a token routes to).

Workload shapes follow the pages' OLMoE-1B-7B runs (64 experts per layer,
Horizon RunMap technical preview, "04 / Resultados") and the 512-expert layer
of the Strata article and of the lucashiago.com.br local-inference explainer
(512 experts, 10 active); the hidden and intermediate sizes, group size and
distributions are the plain readings recorded with the design notes.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np

# tensor ids for the spawn key
T_X = 1          # activations x ~ N(0, 1)
T_ROUTER = 2     # router weights ~ N(0, 0.02)
T_EXPERT = 3     # routed expert weights ~ N(0, 0.02), fp32 before quantisation
T_SHARED = 4     # shared (non-routed) expert weights ~ N(0, 0.02), fp16
T_ZIPF = 5       # per-layer rank permutation for the Zipf logit bias
T_PROMPT = 6     # partial-residency token streams (prompt, token)
T_RESID = 7      # explicit residual input for single-layer cases
T_SGATE = 8      # shared-expert gate vector ~ N(0, 0.02), fp16


@dataclass(frozen=True)
class MoEConfig:
    """One synthetic workload.  Sizes: H hidden, E experts, k top-k,
    I expert intermediate size, g INT4 group size along K, Is shared-expert
    intermediate size (0 = no shared expert)."""
    cid: int
    name: str
    H: int
    E: int
    k: int
    I: int
    g: int
    T: tuple = (1,)
    layers: int = 1
    steps: int = 1
    Is: int = 0
    shared_gate: bool = False
    zipf_s: float = 0.0
    residual: bool = False
    renorm: bool = False
    # partial residency
    capacity: int = 0
    spares: int = 0
    prompts: int = 0
    blocks: int = 0
    tokens_per_prompt: int = 0
    warmup_tokens: int = 0
    extra: dict = field(default_factory=dict)


TINY = MoEConfig(1, "tiny", H=256, E=8, k=2, I=512, g=64, T=(16,))
OLMOE_DECODE = MoEConfig(2, "olmoe_decode", H=2048, E=64, k=8, I=1024, g=128,
                         T=(1,), layers=16, steps=128, residual=True)
OLMOE_BATCHED = MoEConfig(3, "olmoe_batched", H=2048, E=64, k=8, I=1024, g=128,
                          T=(64, 512, 4096))
E512 = MoEConfig(4, "e512_shared", H=2048, E=512, k=10, I=512, g=128,
                 T=(1, 256, 4096), Is=512, zipf_s=1.1)
PARTIAL = MoEConfig(5, "olmoe_partial", H=2048, E=64, k=8, I=1024, g=128,
                    T=(1,), layers=16, residual=True, zipf_s=1.0,
                    capacity=30, spares=8, prompts=12, blocks=3,
                    tokens_per_prompt=128, warmup_tokens=64)

# The 60-expert top-4 model family of the technical preview's residency table
# (top4-fused-v1 rows).  The pages print no layer shape for it; these sizes are
# the published Qwen1.5-MoE-A2.7B architecture (hidden 2048, 60 routed experts
# of intermediate 1408, top-4 without renormalisation, one shared expert of
# intermediate 5632 scaled by a per-token sigmoid gate).
QWEN = MoEConfig(6, "qwen_gated_shared", H=2048, E=60, k=4, I=1408, g=128,
                 T=(1, 256, 4096), Is=5632, shared_gate=True)

CONFIGS = {c.cid: c for c in (TINY, OLMOE_DECODE, OLMOE_BATCHED, E512, PARTIAL, QWEN)}


def rng_for(cid: int, tensor: int, layer: int = 0, expert: int = 0,
            step: int = 0, seed: int = 0) -> np.random.Generator:
    return np.random.default_rng(
        np.random.SeedSequence(seed, spawn_key=(cid, tensor, layer, expert, step)))


def _normal(rng, shape, std):
    a = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a.reshape(shape)


def gen_x(cfg: MoEConfig, T: int, step: int = 0, layer: int = 0,
          tensor: int = T_X) -> np.ndarray:
    """Activations [T, H] as float16 (drawn fp32 N(0,1), rounded by numpy)."""
    return _normal(rng_for(cfg.cid, tensor, layer, T, step), (T, cfg.H), 1.0
                   ).astype(np.float16)


def gen_router(cfg: MoEConfig, layer: int = 0) -> np.ndarray:
    """Router weights [E, H] float16, N(0, 0.02)."""
    return _normal(rng_for(cfg.cid, T_ROUTER, layer), (cfg.E, cfg.H), 0.02
                   ).astype(np.float16)


def gen_expert(cfg: MoEConfig, layer: int, e: int):
    """Full-precision weights of routed expert e: (gate [I,H], up [I,H],
    down [H,I]) float32 ~ N(0, 0.02).  Quantising them is the consumer's job."""
    rng = rng_for(cfg.cid, T_EXPERT, layer, e)
    wg = _normal(rng, (cfg.I, cfg.H), 0.02)
    wu = _normal(rng, (cfg.I, cfg.H), 0.02)
    wd = _normal(rng, (cfg.H, cfg.I), 0.02)
    return wg, wu, wd


def gen_experts(cfg: MoEConfig, layer: int, experts=None, workers: int | None = None):
    """Generate several experts of one layer in parallel threads (numpy's
    generators release the GIL).  Yields (e, (wg, wu, wd)) in expert order."""
    if experts is None:
        experts = range(cfg.E)
    experts = list(experts)
    workers = workers or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(workers) as ex:
        for e, w in zip(experts, ex.map(lambda e: gen_expert(cfg, layer, e), experts)):
            yield e, w


def gen_shared(cfg: MoEConfig):
    """Shared-expert fp16 weights (gate [Is,H], up [Is,H], down [H,Is])."""
    rng = rng_for(cfg.cid, T_SHARED)
    wg = _normal(rng, (cfg.Is, cfg.H), 0.02).astype(np.float16)
    wu = _normal(rng, (cfg.Is, cfg.H), 0.02).astype(np.float16)
    wd = _normal(rng, (cfg.H, cfg.Is), 0.02).astype(np.float16)
    return wg, wu, wd


def gen_shared_gate(cfg: MoEConfig) -> np.ndarray:
    """Shared-expert gate vector [H] fp16, N(0, 0.02)."""
    return _normal(rng_for(cfg.cid, T_SGATE), (cfg.H,), 0.02).astype(np.float16)


def zipf_bias(cfg: MoEConfig, layer: int = 0, s: float | None = None) -> np.ndarray | None:
    """Per-expert router logit bias giving a Zipf(s) skew: expert e of layer l
    gets rank r_l(e) in 1..E from a seeded permutation and bias -s*ln(r), so
    softmax(bias) is the Zipf pmf r^-s / H_{E,s}.  None when s == 0 (no skew,
    the uniform case of the explainer's cache simulation)."""
    s = cfg.zipf_s if s is None else s
    if s == 0.0:
        return None
    perm = rng_for(cfg.cid, T_ZIPF, layer).permutation(cfg.E)
    rank = np.empty(cfg.E, dtype=np.int64)
    rank[perm] = np.arange(1, cfg.E + 1)
    return np.array([-s * math.log(r) for r in rank], dtype=np.float64).astype(np.float32)


def gen_prompt_token(cfg: MoEConfig, prompt: int, token: int) -> np.ndarray:
    """Input x_0 [1, H] fp16 of token `token` of prompt `prompt` (partial
    residency streams).  Prompt -1 is the warmup stream."""
    return _normal(rng_for(cfg.cid, T_PROMPT, prompt + 1, 0, token), (1, cfg.H), 1.0
                   ).astype(np.float16)


def gen_residual(cfg: MoEConfig, T: int) -> np.ndarray:
    return _normal(rng_for(cfg.cid, T_RESID, 0, T), (T, cfg.H), 1.0).astype(np.float16)
