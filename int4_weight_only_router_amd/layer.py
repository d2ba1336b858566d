"""Plumbing around the C ABI: device buffers (torch) and the call sequence of
one MoE layer -- route, permute, routed expert FFN, optional shared expert,
combine.  No arithmetic happens here; every step is a libmoe_w4a16 call on
the given stream.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _abi as A


def load_experts(weights, H, I, group, device="cuda", stream=None, fmt=A.MOE_FMT_SYM):
    """Quantise and prepack experts on the device.

    weights: iterable of (wg [I,H], wu [I,H], wd [H,I]) float32 arrays
    (numpy or torch).  Returns a uint8 device tensor [n, blob_bytes] in the
    device layout (and the canonical blobs).  Quantisation and prepacking run
    in the library's kernels; fmt is MOE_FMT_SYM or MOE_FMT_ZP.
    """
    weights = list(weights)
    n = len(weights)
    _, total = A.moe_blob_layout_fmt(H, I, group, fmt)
    dev = torch.empty((n, total), dtype=torch.uint8, device=device)
    canon = torch.empty((n, total), dtype=torch.uint8, device=device)
    wg = torch.empty((n, I, H), dtype=torch.float32, device=device)
    wu = torch.empty((n, I, H), dtype=torch.float32, device=device)
    wd = torch.empty((n, H, I), dtype=torch.float32, device=device)
    for e, (g_, u_, d_) in enumerate(weights):
        wg[e].copy_(torch.as_tensor(g_))
        wu[e].copy_(torch.as_tensor(u_))
        wd[e].copy_(torch.as_tensor(d_))
    A.moe_quantize_experts_fmt(wg, wu, wd, n, H, I, group, fmt, canon, stream)
    A.moe_prepack_experts_fmt(canon, n, H, I, group, fmt, dev, stream)
    return dev, canon


def blob_table(blobs: torch.Tensor) -> torch.Tensor:
    """Device array of per-expert blob addresses for a [E, bytes] tensor."""
    E, nbytes = blobs.shape
    base = blobs.data_ptr()
    return torch.tensor([base + e * nbytes for e in range(E)], dtype=torch.int64,
                        device=blobs.device)


@dataclass
class LayerBuffers:
    T: int
    regime: int
    y_dtype: int
    y_slices: int
    topk_idx: torch.Tensor
    topk_w: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    perm: torch.Tensor
    inv_perm: torch.Tensor
    perm_ws: torch.Tensor | None
    y: torch.Tensor
    ffn_ws: torch.Tensor | None
    shared_out: torch.Tensor | None
    shared_ws: torch.Tensor | None
    out: torch.Tensor


class MoELayer:
    """One W4A16 MoE layer resident on the device."""

    def __init__(self, H, I, E, k, group, router, table, bias=None, shared=None,
                 renorm=False, device="cuda", shared_gate=None, overlap_shared=False,
                 fmt=A.MOE_FMT_SYM):
        self.H, self.I, self.E, self.k, self.g = H, I, E, k, group
        self.fmt = fmt                  # blob format of the routed experts
        self.router = router            # fp16 [E, H] device
        self.table = table              # int64 [E] device (blob addresses)
        self.bias = bias                # fp32 [E] device or None
        self.shared = shared            # (wg, wu, wd) fp16 device or None
        self.shared_gate = shared_gate  # fp16 [H] device or None (sigmoid-gated shared)
        # run the shared expert on a side stream next to routing + routed FFN
        self.overlap_shared = overlap_shared
        if shared_gate is not None and shared is None:
            raise ValueError("a shared-expert gate needs a shared expert")
        self.flags = A.MOE_RENORM if renorm else 0
        self.device = device

    def buffers(self, T, regime=A.MOE_REGIME_AUTO, partial_order=True) -> LayerBuffers:
        """partial_order: decode partials in partial-major column order, which
        the fused combine + next route reads in whole lines."""
        d = self.device
        r, ydt, ysl, ffn_ws = A.moe_expert_ffn_plan(T, self.H, self.I, self.E, self.k, self.g,
                                                    regime)
        if r == A.MOE_REGIME_DECODE:
            # decode partials straight in token order: the combine then reads
            # them without inv_perm (one dependent round trip less)
            r |= A.MOE_Y_TOKEN_ORDER
            if partial_order and (self.H // 8 <= 64 or (self.H // 8) % 64 == 0):
                r |= A.MOE_Y_PARTIAL_ORDER
                ydt = A.moe_expert_ffn_plan(T, self.H, self.I, self.E, self.k, self.g, r)[1]
        if self.fmt == A.MOE_FMT_ZP:
            r |= A.MOE_W4_ZERO_POINT
        # route/permute scratch; zero-filled once (the fused router keeps an
        # atomic ticket in it)
        pws = max(A.moe_permute_workspace_bytes(T, self.k, self.E),
                  A.moe_route_permute_workspace_bytes(T, self.k, self.E),
                  A.moe_combine_route_permute_workspace_bytes(T, self.k, self.E))
        n = T * self.k
        ytype = torch.float16 if ydt == A.MOE_DTYPE_F16 else torch.float32
        sh_out = sh_ws = None
        if self.shared is not None:
            Is = self.shared[0].shape[0]
            sh_out = torch.empty((T, self.H), dtype=torch.float32, device=d)
            # zero-filled once: the split-K reduction keeps arrival counters
            # in it and leaves them zero after every call
            sh_ws = torch.zeros(max(1, A.moe_shared_ffn_workspace_bytes(T, self.H, Is)),
                                dtype=torch.uint8, device=d)
        return LayerBuffers(
            T=T, regime=r, y_dtype=ydt, y_slices=ysl,
            topk_idx=torch.empty((T, self.k), dtype=torch.int32, device=d),
            topk_w=torch.empty((T, self.k), dtype=torch.float32, device=d),
            counts=torch.empty(self.E, dtype=torch.int32, device=d),
            offsets=torch.empty(self.E + 1, dtype=torch.int32, device=d),
            perm=torch.empty(max(n, 1), dtype=torch.int32, device=d),
            inv_perm=torch.empty(max(n, 1), dtype=torch.int32, device=d),
            perm_ws=torch.zeros(pws, dtype=torch.uint8, device=d) if pws else None,
            y=torch.empty((ysl, max(n, 1), self.H), dtype=ytype, device=d),
            ffn_ws=torch.empty(ffn_ws, dtype=torch.uint8, device=d) if ffn_ws else None,
            shared_out=sh_out, shared_ws=sh_ws,
            out=torch.empty((T, self.H), dtype=torch.float16, device=d),
        )

    def route_permute(self, x, b: LayerBuffers, stream=None, fused=True):
        T = b.T
        nws = 0 if b.perm_ws is None else b.perm_ws.numel()
        if fused:
            A.moe_route_permute(x, self.router, self.bias, T, self.H, self.E, self.k,
                                self.flags, b.topk_idx, b.topk_w, b.counts, b.offsets, b.perm,
                                b.inv_perm, b.perm_ws, nws, stream)
            return
        A.moe_route(x, self.router, self.bias, T, self.H, self.E, self.k, self.flags,
                    b.topk_idx, b.topk_w, b.perm_ws, nws, stream)
        A.moe_permute(b.topk_idx, T, self.k, self.E, b.counts, b.offsets, b.perm, b.inv_perm,
                      b.perm_ws, nws, stream)

    def shared_ffn(self, x, b: LayerBuffers, stream=None):
        wg, wu, wd = self.shared
        A.moe_shared_ffn_f16(x, wg, wu, wd, b.T, self.H, wg.shape[0], b.shared_out,
                             b.shared_ws, b.shared_ws.numel(), stream)

    def experts(self, x, b: LayerBuffers, table=None, stream=None, shared=True):
        A.moe_expert_ffn_w4a16(x, b.perm, b.offsets, self.table if table is None else table,
                               b.T, self.H, self.I, self.E, self.k, self.g, b.regime, b.y,
                               b.y_dtype, b.y_slices, b.ffn_ws,
                               0 if b.ffn_ws is None else b.ffn_ws.numel(), stream)
        if shared and self.shared is not None:
            self.shared_ffn(x, b, stream)

    def combine(self, b: LayerBuffers, residual=None, out=None, stream=None, x=None):
        """x (the layer input) is needed only when the shared expert is gated."""
        out = b.out if out is None else out
        inv = None if b.regime & A.MOE_Y_TOKEN_ORDER else b.inv_perm
        if self.shared_gate is not None:
            if x is None:
                raise ValueError("the gated shared expert needs the layer input x")
            A.moe_combine_gated(b.y, b.y_dtype, b.y_slices, inv, b.topk_w, b.shared_out,
                                x, self.shared_gate, residual, b.T, self.H, self.k, out, stream)
            return out
        A.moe_combine(b.y, b.y_dtype, b.y_slices, inv, b.topk_w, b.shared_out, residual,
                      b.T, self.H, self.k, out, stream)
        return out

    def combine_route_next(self, b: LayerBuffers, nxt: "MoELayer", b_next: LayerBuffers,
                           residual=None, out=None, stream=None, x=None):
        """This layer's combine into `out` fused with the next layer's route +
        permute of `out` into b_next (moe_combine_route_permute: one launch for a
        decode token of at most 64 experts, else the two calls)."""
        if nxt.H != self.H or b_next.T != b.T:
            raise ValueError("the next layer must have the same H and batch")
        out = b.out if out is None else out
        inv = None if b.regime & A.MOE_Y_TOKEN_ORDER else b.inv_perm
        gate = self.shared_gate
        if gate is not None and x is None:
            raise ValueError("the gated shared expert needs the layer input x")
        nws = 0 if b_next.perm_ws is None else b_next.perm_ws.numel()
        A.moe_combine_route_permute(b.y, b.y_dtype, b.y_slices, inv, b.topk_w, b.shared_out,
                                    x if gate is not None else None, gate, residual, b.T,
                                    self.H, self.k, out, nxt.router, nxt.bias, nxt.E, nxt.k,
                                    nxt.flags, b_next.topk_idx, b_next.topk_w, b_next.counts,
                                    b_next.offsets, b_next.perm, b_next.inv_perm, b_next.perm_ws,
                                    nws, stream)
        return out

    def split_route_ok(self, b: LayerBuffers, nxt: "MoELayer") -> bool:
        """Whether this layer's combine can hand the next layer only its logit
        partials (moe_combine_route_partials): one decode token, at most 64
        experts in the next layer, fp32 slice partials here."""
        return (b.T == 1 and nxt.E <= 64 and nxt.H == self.H and b.y_slices > 1 and
                b.y_dtype in (A.MOE_DTYPE_F32, A.MOE_DTYPE_F32_PM))

    def combine_partials_next(self, b: LayerBuffers, nxt: "MoELayer", parts,
                              residual=None, out=None, stream=None, x=None):
        """This layer's combine into `out` plus the next layer's logit partials
        of `out` into `parts` (fp32, moe_logit_partials_bytes()), which
        nxt.experts_routed then routes from."""
        out = b.out if out is None else out
        inv = None if b.regime & A.MOE_Y_TOKEN_ORDER else b.inv_perm
        gate = self.shared_gate
        if gate is not None and x is None:
            raise ValueError("the gated shared expert needs the layer input x")
        A.moe_combine_route_partials(b.y, b.y_dtype, b.y_slices, inv, b.topk_w, b.shared_out,
                                     x if gate is not None else None, gate, residual, b.T,
                                     self.H, self.k, out, nxt.router, nxt.E, parts, stream)
        return out

    def route_from_partials_ok(self, b: LayerBuffers) -> bool:
        """Whether this layer's expert launch can route from logit partials
        (moe_expert_ffn_w4a16_routed): one decode token, at most 64 experts."""
        return b.T == 1 and self.E <= 64 and b.regime & 0xFF == A.MOE_REGIME_DECODE

    def logit_partials(self, x, parts, stream=None):
        """This layer's logit partials of an input row in hand (the first
        layer of a stack) into `parts`, for experts_routed."""
        A.moe_logit_partials(x, self.router, 1, self.H, self.E, parts, stream)

    def experts_routed(self, x, b: LayerBuffers, parts, stream=None, shared=True):
        """Routing from the logit partials of the previous layer's combine and
        the routed experts in one launch (moe_expert_ffn_w4a16_routed): fills
        b's routing arrays and y as route_permute + experts would."""
        A.moe_expert_ffn_w4a16_routed(x, parts, self.bias, self.E, self.k, self.flags,
                                      b.topk_idx, b.topk_w, b.counts, b.offsets, b.perm,
                                      b.inv_perm, self.table, b.T, self.H, self.I, self.g,
                                      b.regime, b.y, b.y_dtype, b.y_slices, stream)
        if shared and self.shared is not None:
            self.shared_ffn(x, b, stream)

    def pool_args(self, b: LayerBuffers, host_ids):
        """PoolLayerArgs for moe_pool_layer_forward with this layer's weights and
        b's buffers; x_f16 / residual_f16 / out_f16 are set per call."""
        if self.shared is not None:
            raise ValueError("pooled layers carry no shared expert")
        z = lambda t: 0 if t is None else t.data_ptr()
        a = A.PoolLayerArgs()
        a.w_router_f16, a.logit_bias = z(self.router), z(self.bias)
        a.T, a.H, a.I, a.k, a.group, a.flags = b.T, self.H, self.I, self.k, self.g, self.flags
        a.topk_idx, a.topk_w, a.counts = z(b.topk_idx), z(b.topk_w), z(b.counts)
        a.offsets, a.perm, a.inv_perm = z(b.offsets), z(b.perm), z(b.inv_perm)
        a.route_ws, a.route_ws_bytes = z(b.perm_ws), 0 if b.perm_ws is None else b.perm_ws.numel()
        a.regime, a.y, a.y_dtype, a.y_slices = b.regime, z(b.y), b.y_dtype, b.y_slices
        a.ffn_ws, a.ffn_ws_bytes = z(b.ffn_ws), 0 if b.ffn_ws is None else b.ffn_ws.numel()
        a.host_ids = host_ids.data_ptr()
        return a

    def _side(self):
        st = getattr(self, "_side_stream", None)
        if st is None:
            st = self._side_stream = torch.cuda.Stream(device=self.device)
        return st

    def forward(self, x, b: LayerBuffers, residual=None, out=None, stream=None,
                overlap_shared=None):
        """One layer.  With overlap_shared (default: the layer's setting) the
        shared expert runs on a side stream, forked at the layer's start and
        joined before the combine: it reads only x, so it overlaps routing and
        the routed experts.  That pays when the shared weights are large
        (60-expert layer, 69 MB: -12% per layer at T = 8..256) and costs when
        they are small (512-expert layer, 6 MB: +17% at T = 1, the shared
        kernels then delay the latency-bound router)."""
        if overlap_shared is None:
            overlap_shared = self.overlap_shared
        if self.shared is None or not overlap_shared or isinstance(stream, int):
            self.route_permute(x, b, stream)
            self.experts(x, b, stream=stream)
            return self.combine(b, residual, out, stream, x=x)
        main = torch.cuda.current_stream(self.device) if stream is None else stream
        side = self._side()
        fork = torch.cuda.Event()
        fork.record(main)
        side.wait_event(fork)
        if not torch.cuda.is_current_stream_capturing():
            x.record_stream(side)
        self.shared_ffn(x, b, side)
        join = torch.cuda.Event()
        join.record(side)
        self.route_permute(x, b, main)
        self.experts(x, b, stream=main, shared=False)
        main.wait_event(join)
        return self.combine(b, residual, out, main, x=x)


def stack_forward(layers, bufs, acts, stream=None, fuse=True, parts=None):
    """Stacked layers with residual connections, x_{l+1} = fp16(x_l + MoE_l(x_l)):
    acts[l] is layer l's input and residual, acts[l + 1] its output.  With
    `fuse`, each layer's combine runs together with the next layer's route +
    permute (MoELayer.combine_route_next); with `parts` as well (fp32 device
    buffer of moe_logit_partials_bytes()), a decode token's combine hands the
    next layer only its logit partials and that layer's expert launch routes
    from them (combine_partials_next + experts_routed), the first layer's
    from moe_logit_partials of its input.  Every form gives the same bits."""
    L = len(layers)
    # routed: this layer's routing is still to be formed from `parts`
    routed = fuse and parts is not None and layers[0].route_from_partials_ok(bufs[0])
    if routed:
        layers[0].logit_partials(acts[0], parts, stream)
    else:
        layers[0].route_permute(acts[0], bufs[0], stream)
    for l, lay in enumerate(layers):
        if l > 0 and not fuse:
            lay.route_permute(acts[l], bufs[l], stream)
        if routed:
            lay.experts_routed(acts[l], bufs[l], parts, stream=stream)
        else:
            lay.experts(acts[l], bufs[l], stream=stream)
        routed = False
        if fuse and l + 1 < L:
            nxt = layers[l + 1]
            if parts is not None and lay.split_route_ok(bufs[l], nxt) and \
                    bufs[l + 1].regime & 0xFF == A.MOE_REGIME_DECODE:
                lay.combine_partials_next(bufs[l], nxt, parts, residual=acts[l],
                                          out=acts[l + 1], stream=stream, x=acts[l])
                routed = True
            else:
                lay.combine_route_next(bufs[l], nxt, bufs[l + 1], residual=acts[l],
                                       out=acts[l + 1], stream=stream, x=acts[l])
        else:
            lay.combine(bufs[l], residual=acts[l], out=acts[l + 1], stream=stream, x=acts[l])
    return acts[L]
