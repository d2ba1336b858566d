"""The C-ABI library loads without a GPU, exports every symbol the header
declares, and rejects bad arguments on the host before launching anything."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import int4_weight_only_router_amd as M
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w4a16.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", txt)))


def test_header_and_binding_agree():
    assert _declared() == sorted(M.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = C.CDLL(M.lib()._name)
    for name in _declared():
        assert hasattr(L, name), name


@pytest.mark.parametrize("H,I,g", [(256, 512, 64), (2048, 1024, 128), (2048, 512, 128),
                                   (512, 192, 32)])
def test_blob_layout_matches_oracle(H, I, g):
    assert M.moe_blob_layout(H, I, g) == O.blob_layout(H, I, g)


def test_plan_regimes():
    # decode: fp32 partials over I/32 slices, no workspace
    assert M.moe_expert_ffn_plan(1, 2048, 1024, 64, 8, 128) == (M.MOE_REGIME_DECODE,
                                                                M.MOE_DTYPE_F32, 32, 0)
    r, dt, sl, ws = M.moe_expert_ffn_plan(4096, 2048, 1024, 64, 8, 128)
    assert (r, dt, sl) == (M.MOE_REGIME_BATCHED, M.MOE_DTYPE_F16, 1)
    assert ws >= 4096 * 8 * 1024 * 2
    r, *_ = M.moe_expert_ffn_plan(1, 2048, 1024, 64, 8, 128, M.MOE_REGIME_BATCHED)
    assert r == M.MOE_REGIME_BATCHED
    # small batch: fp16 y, h in the workspace
    r, dt, sl, ws = M.moe_expert_ffn_plan(8, 2048, 1024, 64, 8, 128)
    assert (r, dt, sl) == (M.MOE_REGIME_SMALL, M.MOE_DTYPE_F16, 1)
    assert ws >= 8 * 8 * 1024 * 2
    assert M.moe_expert_ffn_plan(32, 2048, 1024, 64, 8, 128)[0] == M.MOE_REGIME_SMALL
    assert M.moe_expert_ffn_plan(33, 2048, 1024, 64, 8, 128)[0] == M.MOE_REGIME_BATCHED
    assert M.moe_expert_ffn_plan(1, 256, 512, 8, 2, 64, M.MOE_REGIME_SMALL)[0] == \
        M.MOE_REGIME_SMALL
    assert M.moe_expert_ffn_plan(32, 2048, 8192, 64, 8, 128)[0] == M.MOE_REGIME_SMALL
    assert M.moe_expert_ffn_plan(4, 2048, 1024, 64, 8, 128)[0] == M.MOE_REGIME_DECODE
    assert M.moe_expert_ffn_plan(5, 2048, 1024, 64, 8, 128)[0] == M.MOE_REGIME_SMALL
    # token-order y: a decode option; the resolved regime comes back without it
    tok = M.MOE_Y_TOKEN_ORDER
    assert M.moe_expert_ffn_plan(1, 2048, 1024, 64, 8, 128, tok) == (M.MOE_REGIME_DECODE,
                                                                     M.MOE_DTYPE_F32, 32, 0)
    assert M.moe_expert_ffn_plan(3, 2048, 1024, 64, 8, 128, M.MOE_REGIME_DECODE | tok)[0] == \
        M.MOE_REGIME_DECODE
    # partial-major decode columns: reported as their own y dtype
    pm = M.MOE_Y_PARTIAL_ORDER
    for H in (256, 512, 1024, 2048):
        assert M.moe_expert_ffn_plan(1, H, 1024, 64, 8, 64, tok | pm) == (
            M.MOE_REGIME_DECODE, M.MOE_DTYPE_F32_PM, 32, 0)


@pytest.mark.parametrize("args,code", [
    ((1, 2048, 1024, 64, 65, 128), M.MOE_EINVAL),        # k > E
    ((1, 2048, 1024, 64, 8, 100), M.MOE_EINVAL),         # g not a multiple of 32
    ((1, 2048, 1000, 64, 8, 8 * 125), M.MOE_EINVAL),     # g does not divide H
    ((1, 1536, 1024, 64, 8, 128), M.MOE_EUNSUPPORTED),   # H outside the envelope
    ((1, 2048, 1056, 64, 8, 32), M.MOE_EUNSUPPORTED),    # I % 64 != 0
    ((1, 2048, 1024, 2048, 8, 128), M.MOE_EUNSUPPORTED),  # E > 1024
    ((1, 2048, 1024, 64, 17, 128), M.MOE_EUNSUPPORTED),  # k > 16
    ((-1, 2048, 1024, 64, 8, 128), M.MOE_EINVAL),        # T < 0
    ((1, 2048, 1024, 64, 8, 128, 4), M.MOE_EINVAL),      # unknown regime
    ((33, 2048, 1024, 64, 8, 128, M.MOE_REGIME_SMALL), M.MOE_EUNSUPPORTED),   # T > 32
    ((64, 2048, 1024, 64, 8, 128, M.MOE_Y_TOKEN_ORDER), M.MOE_EUNSUPPORTED),  # token order
    ((1, 2048, 1024, 64, 8, 128, M.MOE_REGIME_BATCHED | M.MOE_Y_TOKEN_ORDER),
     M.MOE_EUNSUPPORTED),                                                     # off decode
    ((64, 2048, 1024, 64, 8, 128, M.MOE_Y_PARTIAL_ORDER), M.MOE_EUNSUPPORTED),  # off decode
])
def test_plan_rejections(args, code):
    with pytest.raises(M.MoEError) as ei:
        M.moe_expert_ffn_plan(*args)
    assert ei.value.code == code
    assert M.moe_last_error()


def test_compute_calls_reject_before_launch():
    # every call below fails validation on the host; no GPU is touched
    with pytest.raises(M.MoEError) as ei:
        M.moe_route(1, 1, None, 4, 2048, 8, 9, 0, 1, 1, stream=0)
    assert ei.value.code == M.MOE_EINVAL
    with pytest.raises(M.MoEError) as ei:
        M.moe_route(1, 1, None, 4, 2048, 8, 2, 4, 1, 1, stream=0)   # unknown flag
    assert ei.value.code == M.MOE_EINVAL
    with pytest.raises(M.MoEError) as ei:
        M.moe_route(1, 1, None, 100, 2048, 64, 8, 0, 1, 1, None, 0, stream=0)  # no logit ws
    assert ei.value.code == M.MOE_ENOMEM
    with pytest.raises(M.MoEError) as ei:
        M.moe_permute(1, 10000, 8, 64, 1, 1, 1, 1, None, 0, stream=0)  # workspace missing
    assert ei.value.code == M.MOE_ENOMEM
    with pytest.raises(M.MoEError) as ei:   # y dtype does not match the plan
        M.moe_expert_ffn_w4a16(1, 1, 1, 1, 1, 2048, 1024, 64, 8, 128, M.MOE_REGIME_DECODE, 1,
                               M.MOE_DTYPE_F16, 1, stream=0)
    assert ei.value.code == M.MOE_EINVAL
    with pytest.raises(M.MoEError) as ei:   # x or y not 16-byte aligned
        M.moe_expert_ffn_w4a16(4096, 1, 1, 1, 1, 2048, 1024, 64, 8, 128, M.MOE_REGIME_DECODE,
                               4096 + 8, M.MOE_DTYPE_F32, 32, stream=0)
    assert ei.value.code == M.MOE_EINVAL and "aligned" in str(ei.value)
    with pytest.raises(M.MoEError) as ei:
        M.moe_expert_ffn_w4a16(4096 + 8, 1, 1, 1, 1, 2048, 1024, 64, 8, 128,
                               M.MOE_REGIME_DECODE, 4096, M.MOE_DTYPE_F32, 32, stream=0)
    assert ei.value.code == M.MOE_EINVAL and "aligned" in str(ei.value)
    with pytest.raises(M.MoEError) as ei:
        M.moe_combine(1, M.MOE_DTYPE_F16, 4, 1, 1, None, None, 1, 2048, 8, 1, stream=0)
    assert ei.value.code == M.MOE_EINVAL
    with pytest.raises(M.MoEError) as ei:   # y not 16-byte aligned
        M.moe_combine(4104, M.MOE_DTYPE_F32, 32, None, 256, None, None, 1, 2048, 8, 512,
                      stream=0)
    assert ei.value.code == M.MOE_EINVAL and "aligned" in str(ei.value)
    with pytest.raises(M.MoEError) as ei:   # overlapping prepack buffers
        M.moe_prepack_experts(4096, 2, 256, 512, 64, 4096 + 256, stream=0)
    assert ei.value.code == M.MOE_EINVAL
    with pytest.raises(M.MoEError) as ei:   # logit partials: two tokens
        M.moe_logit_partials(4096, 8192, 2, 2048, 64, 4096, stream=0)
    assert ei.value.code == M.MOE_EUNSUPPORTED
    with pytest.raises(M.MoEError) as ei:   # more than 64 experts
        M.moe_logit_partials(4096, 8192, 1, 2048, 65, 4096, stream=0)
    assert ei.value.code == M.MOE_EUNSUPPORTED
    with pytest.raises(M.MoEError) as ei:   # x not 16-byte aligned
        M.moe_logit_partials(4096 + 2, 8192, 1, 2048, 64, 4096, stream=0)
    assert ei.value.code == M.MOE_EINVAL and "aligned" in str(ei.value)
    with pytest.raises(M.MoEError) as ei:   # H not instantiated
        M.moe_logit_partials(4096, 8192, 1, 768, 64, 4096, stream=0)
    assert ei.value.code == M.MOE_EUNSUPPORTED
    # T = 0 is a valid no-op for the routed FFN and combine
    M.moe_expert_ffn_w4a16(None, None, None, None, 0, 2048, 1024, 64, 8, 128,
                           M.MOE_REGIME_DECODE, None, M.MOE_DTYPE_F32, 32, stream=0)
    M.moe_combine(None, M.MOE_DTYPE_F32, 32, None, None, None, None, 0, 2048, 8, None, stream=0)


def test_pool_create_rejects_bad_profiles():
    cfg = M.PoolConfig(layers=1, experts=8, topk=2, capacity=1, spares=2, decay_shift=3,
                       expert_bytes=256)
    with pytest.raises(M.MoEError) as ei:
        M.moe_pool_create(cfg, [1] * 8)
    assert ei.value.code == M.MOE_ECAPACITY
    cfg.capacity, cfg.spares = 4, 1          # too few spares
    with pytest.raises(M.MoEError) as ei:
        M.moe_pool_create(cfg, [1] * 8)
    assert ei.value.code == M.MOE_ECAPACITY


def test_route_workspace_sizes():
    # one-workgroup router up to 8 tokens needs no scratch; above, T x E fp32 logits
    assert M.moe_route_workspace_bytes(8, 512) == 0
    assert M.moe_route_workspace_bytes(9, 64) >= 9 * 64 * 4
    assert M.moe_route_workspace_bytes(4096, 512) == 4096 * 512 * 4
    # route + permute above 8 tokens: logits, then the permutation's scratch
    assert (M.moe_route_permute_workspace_bytes(4096, 8, 64)
            >= M.moe_route_workspace_bytes(4096, 64) + M.moe_permute_workspace_bytes(4096, 8, 64))


def test_pool_layer_forward_rejects_null_arguments():
    # validation happens on the host before anything is launched
    args = M.PoolLayerArgs()
    with pytest.raises(M.MoEError) as ei:
        M.moe_pool_layer_forward(None, 0, args, stream=0)
    assert ei.value.code == M.MOE_EINVAL


@pytest.mark.parametrize("H,I,g,fmt", [(256, 512, 64, 0), (256, 512, 64, 1), (512, 192, 32, 1),
                                       (1024, 128, 128, 0)])
def test_host_prepack_matches_layout_and_round_trips(H, I, g, fmt):
    """moe_prepack_expert_host renders an oracle-packed canonical blob into the
    documented device layout (checked against an independent numpy
    rendering), and moe_unpack_expert_host inverts it exactly."""
    import moe_inputs as MI
    from tests.layout_util import numpy_prepack
    cfg = MI.MoEConfig(96, "hp", H=H, E=1, k=1, I=I, g=g)
    canon = O.pack_expert(*MI.gen_expert(cfg, 0, 0), g, fmt)
    dev = np.full_like(canon, 0xAB)
    M.moe_prepack_expert_host(canon, H, I, g, fmt, dev)
    assert np.array_equal(dev, numpy_prepack(canon, H, I, g, fmt))
    back = np.full_like(canon, 0xCD)
    M.moe_unpack_expert_host(dev, H, I, g, fmt, back)
    assert np.array_equal(back, canon)
    with pytest.raises(M.MoEError):
        M.moe_prepack_expert_host(canon, H, I, 48, fmt, dev)
    with pytest.raises(M.MoEError):
        M.moe_prepack_expert_host(canon, H, I, g, 7, dev)
