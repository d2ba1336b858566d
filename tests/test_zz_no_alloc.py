"""moe_route_permute_noalloc (the library's own scratch, no allocation)
against moe_route_permute with a caller workspace: identical routing and
permutation bits, on consecutive calls that share the scratch, the later
ones smaller (the batched two-launch path, then the fused one-launch path),
and size rejection before any launch."""
import ctypes as C

import numpy as np
import pytest
import torch

import int4_weight_only_router_amd as M
import moe_inputs as MI
from tests.gpu_util import DEV, f16, say

pytestmark = pytest.mark.gpu


def _outs(T, k, E):
    n = max(1, T * k)
    return [torch.full((T, k), -7, dtype=torch.int32, device=DEV),
            torch.full((T, k), -7.0, dtype=torch.float32, device=DEV),
            torch.full((E,), -7, dtype=torch.int32, device=DEV),
            torch.full((E + 1,), -7, dtype=torch.int32, device=DEV),
            torch.full((n,), -7, dtype=torch.int32, device=DEV),
            torch.full((n,), -7, dtype=torch.int32, device=DEV)]


def _both(cfg, T, step):
    x = f16(MI.gen_x(cfg, T, step=step))
    wr = f16(MI.gen_router(cfg))
    b = MI.zipf_bias(cfg)
    bias = None if b is None else torch.from_numpy(b).to(DEV)
    ref = _outs(T, cfg.k, cfg.E)
    wsb = M.moe_route_permute_workspace_bytes(T, cfg.k, cfg.E)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=DEV)
    M.moe_route_permute(x, wr, bias, T, cfg.H, cfg.E, cfg.k, 0, *ref, ws, wsb)
    got = _outs(T, cfg.k, cfg.E)
    M.moe_route_permute_noalloc(x, wr, bias, T, cfg.H, cfg.E, cfg.k, 0, *got)
    torch.cuda.synchronize()
    n = T * cfg.k
    for name, a, r in zip(("idx", "w", "counts", "offsets", "perm", "inv_perm"), got, ref):
        a, r = a.cpu().numpy(), r.cpu().numpy()
        if name in ("perm", "inv_perm"):
            a, r = a[:n], r[:n]
        assert np.array_equal(a.view(np.uint8), r.view(np.uint8)), (cfg.name, T, name)


@pytest.mark.parametrize("cfg,Ts", [(MI.E512, (4096, 300, 4, 1)), (MI.OLMOE_DECODE, (512, 1, 1)),
                                    (MI.TINY, (16, 3))], ids=lambda v: getattr(v, "name", str(v)))
def test_noalloc_matches_workspace_entry_on_consecutive_calls(cfg, Ts):
    for i, T in enumerate(Ts):
        say("noalloc %s T=%d" % (cfg.name, T))
        _both(cfg, T, step=20 + i)


def test_noalloc_rejects_oversized_shapes_before_launch():
    cfg = MI.OLMOE_DECODE
    T, E, k = 8192, 1024, 16     # 4*T*E bytes of logits alone: 32 MiB
    need = M.moe_route_permute_workspace_bytes(T, k, E)
    assert need > 16 << 20
    x = torch.zeros((1, cfg.H), dtype=torch.float16, device=DEV)
    wr = torch.zeros((1, cfg.H), dtype=torch.float16, device=DEV)
    o = torch.zeros(16, dtype=torch.int32, device=DEV)
    L = M.lib()
    rc = L.moe_route_permute_noalloc(x.data_ptr(), wr.data_ptr(), None, T, cfg.H, E, k, 0,
                                     o.data_ptr(), o.data_ptr(), o.data_ptr(), o.data_ptr(),
                                     o.data_ptr(), o.data_ptr(), None)
    assert rc == M.MOE_ENOMEM and "16777216" in M.moe_last_error()
    torch.cuda.synchronize()
    assert torch.count_nonzero(o) == 0     # nothing was launched
