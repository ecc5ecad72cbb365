"""The routed NVFP4 W4A4 MoE layer as one object: the C-ABI calls in order.

forward(x):  moe_route_quantize -> moe_nvfp4_gate_up_swiglu ->
             moe_nvfp4_down_scatter -> moe_combine (moe_combine_reap with REAP)
block output: moe_shared_expert on a second stream, joined by moe_combine_block
(the two FFN calls are the stages of moe_nvfp4_grouped_ffn)
All buffers for a given token count are allocated once and reused, so a
forward pass enqueues only kernels on the current stream.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import ops


@dataclass
class LayerOut:
    y: torch.Tensor
    route: ops.RouteOut
    x_codes: torch.Tensor
    x_scales: torch.Tensor
    pair_out: torch.Tensor  # FP16 [T*k, H]: pair row p = pair_out[p] * pair_scale[p]
    pair_scale: torch.Tensor  # FP32 [T*k], powers of two
    pair_sqnorm: Optional[torch.Tensor]
    saliency: Optional[torch.Tensor]
    shared_out: Optional[torch.Tensor] = None  # the shared expert's FP32 output (block=True)
    h_codes: Optional[torch.Tensor] = None  # re-quantized hidden state [T*k, I/2], rows in sorted-pair order
    h_scales: Optional[torch.Tensor] = None  # its E4M3 block scales [T*k, I/16]


class NVFP4MoELayer:
    def __init__(self, w_router_bf16, bias, k: int, rsf: float, x_gs, h_gs, w13_codes, w13_scales, w13_gs,
                 w2_codes, w2_scales, w2_gs):
        self.w_router = w_router_bf16
        self.bias = bias
        self.k = int(k)
        self.rsf = float(rsf)
        self.x_gs = x_gs.reshape(1)
        self.h_gs = h_gs
        self.w13 = (w13_codes, w13_scales, w13_gs)
        self.w2 = (w2_codes, w2_scales, w2_gs)
        self.E, two_i, h_half = w13_codes.shape
        self.H, self.I = 2 * h_half, two_i // 2
        self.device = w13_codes.device
        self._bufs: dict = {}
        self.keep_ids = None  # set on a layer made by prune(): its experts' ids in the unpruned layer
        self.shared = None  # (w13 [2I_s, H], w2 [H, I_s]) BF16 of the shared expert, if attached
        self._side = None  # stream the shared expert runs on, beside the routed path

    def set_shared_expert(self, w13_bf16: torch.Tensor, w2_bf16: torch.Tensor) -> None:
        """Attach the BF16 shared expert (gate rows then up rows in w13); forward(block=True) adds it."""
        self.shared = (w13_bf16, w2_bf16)

    @classmethod
    def from_bf16(cls, w_router_bf16, bias, k, rsf, x_gs, h_gs, w13_bf16, w2_bf16):
        """Quantize BF16 expert weights with the library (offline RTN, per expert Linear).

        w13_bf16 [E, 2I, H] (gate rows then up rows), w2_bf16 [E, H, I]."""
        E, two_i, H = w13_bf16.shape
        I = two_i // 2
        c13, s13, g13 = ops.nvfp4_quantize_weights(w13_bf16.view(2 * E, I, H))
        c2, s2, g2 = ops.nvfp4_quantize_weights(w2_bf16)
        return cls(w_router_bf16, bias, k, rsf, x_gs, h_gs, c13.view(E, 2 * I, H // 2),
                   s13.view(E, 2 * I // 16, H // 128, 16, 8), g13.view(E, 2), c2, s2, g2)

    def _buffers(self, T: int, reap: bool, out_dtype: torch.dtype, block: bool = False):
        key = (T, reap, out_dtype, block)
        b = self._bufs.get(key)
        if b is None:
            d, E, H, I, k = self.device, self.E, self.H, self.I, self.k
            b = dict(
                route=ops.RouteOut(torch.empty((T, k), dtype=torch.int32, device=d),
                                   torch.empty((T, k), dtype=torch.float32, device=d),
                                   torch.empty((E,), dtype=torch.int32, device=d),
                                   torch.empty((E + 1,), dtype=torch.int32, device=d),
                                   torch.empty((T * k,), dtype=torch.int32, device=d)),
                route_ws=torch.empty((max(ops.moe_route_workspace_bytes(T, H, E, k), 1),), dtype=torch.uint8, device=d),
                x_codes=torch.empty((T, H // 2), dtype=torch.uint8, device=d),
                x_scales=torch.empty((T, H // 16), dtype=torch.uint8, device=d),
                pair_out=torch.empty((T * k, H), dtype=torch.float16, device=d),
                pair_scale=torch.empty((T * k,), dtype=torch.float32, device=d),
                pair_sqnorm=torch.empty((T * k,), dtype=torch.float32, device=d) if reap else None,
                h_codes=torch.empty((T * k, I // 2), dtype=torch.uint8, device=d),
                h_scales=torch.empty((T * k, I // 16), dtype=torch.uint8, device=d),
                ffn_ws=torch.empty((max(ops.moe_ffn_stage_workspace_bytes(T, k, E, H, I), 1),), dtype=torch.uint8,
                                   device=d),
                y=torch.empty((T, H), dtype=out_dtype, device=d),
                saliency=torch.empty((E,), dtype=torch.float32, device=d) if reap else None,
            )
            if block:
                Is = self.shared[1].shape[1]
                b["shared_out"] = torch.empty((T, H), dtype=torch.float32, device=d)
                b["shared_ws"] = torch.empty((max(ops.moe_shared_workspace_bytes(T, H, Is), 1),), dtype=torch.uint8,
                                             device=d)
                b["ev_in"] = torch.cuda.Event()
                b["ev_shared"] = torch.cuda.Event()
            self._bufs[key] = b
        return b

    def prune(self, saliency: torch.Tensor, n_keep: int) -> "NVFP4MoELayer":
        """REAP one-shot pruning: a new layer with the n_keep highest-saliency experts.

        The router rows, the bias and every expert tensor are sliced to the
        kept experts, in ascending original index ("K-EXAONE-152B-A23B-REAP-80E-BF16"
        model card, "Pruning Setup").  The kept ids are in ``.keep_ids``."""
        return self.take_experts(ops.reap_prune_select(saliency, n_keep))

    def take_experts(self, keep_ids: torch.Tensor) -> "NVFP4MoELayer":
        """A new layer whose expert i is this layer's expert keep_ids[i] (INT32 on the device):
        router rows, bias, calibrated h global scales and every expert tensor gathered."""
        g = lambda t: ops.moe_gather_experts(t, keep_ids)  # noqa: E731
        out = NVFP4MoELayer(g(self.w_router), g(self.bias), self.k, self.rsf, self.x_gs, g(self.h_gs),
                            *(g(t) for t in self.w13), *(g(t) for t in self.w2))
        out.keep_ids = keep_ids
        out.shared = self.shared  # the shared expert is kept whole
        return out

    STAGES = ("route_quantize", "gate_up", "down", "combine_reap")

    def forward(self, x_bf16: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16, reap: bool = False,
                events: Optional[list] = None, block: bool = False) -> LayerOut:
        """One layer pass.  If `events` is a list of len(STAGES) + 1 timing events
        (entries may be None), they are recorded on the current stream around each stage.

        block=True returns the MoE block output (routed combine + shared expert):
        the shared expert runs on a second stream (default priority) while the
        routed path runs on the current one, and the combine waits for both."""
        T = x_bf16.shape[0]
        if block and self.shared is None:
            raise ValueError("block=True needs a shared expert (set_shared_expert)")
        b = self._buffers(T, reap, out_dtype, block)
        def mark(i):  # record event i if one was given for that position
            if events is not None and events[i] is not None:
                events[i].record()

        if block:
            cur = torch.cuda.current_stream(self.device)
            if self._side is None:
                self._side = torch.cuda.Stream(self.device)
            b["ev_in"].record(cur)
            self._side.wait_event(b["ev_in"])
            ops.moe_shared_expert(x_bf16, *self.shared, out=b["shared_out"], workspace=b["shared_ws"],
                                  stream=self._side)
            b["ev_shared"].record(self._side)
        mark(0)
        # routing and the NVFP4 quantization of x in one pass over x
        r, _, _ = ops.moe_route_quantize(x_bf16, self.w_router, self.bias, self.k, self.rsf, self.x_gs,
                                         out=b["route"], x_codes=b["x_codes"], x_scales=b["x_scales"],
                                         workspace=b["route_ws"])
        mark(1)
        # the two stages of moe_nvfp4_grouped_ffn, called separately so each can be timed
        ops.moe_nvfp4_gate_up_swiglu(b["x_codes"], b["x_scales"], self.x_gs, *self.w13, self.h_gs, self.k,
                                     r.expert_offsets, r.sorted_pair_ids, b["h_codes"], b["h_scales"],
                                     workspace=b["ffn_ws"])
        mark(2)
        ops.moe_nvfp4_down_scatter(b["h_codes"], b["h_scales"], self.h_gs, T, *self.w2, self.k, r.expert_offsets,
                                   r.sorted_pair_ids, r.topk_w, pair_out=b["pair_out"], pair_scale=b["pair_scale"],
                                   pair_sqnorm=b["pair_sqnorm"] if reap else None, workspace=b["ffn_ws"])
        mark(3)
        sal = None
        if block:
            torch.cuda.current_stream(self.device).wait_event(b["ev_shared"])
            ops.moe_combine_block(b["pair_out"], b["pair_scale"], b["shared_out"], T, self.k, out_dtype, y=b["y"])
            if reap:
                sal = ops.reap_saliency(b["pair_sqnorm"], r.topk_w, r.expert_offsets, r.sorted_pair_ids, T, self.k,
                                        self.E, out=b["saliency"])
        elif reap:  # the combine and the saliency in one launch
            _, sal = ops.moe_combine_reap(b["pair_out"], b["pair_scale"], T, self.k, b["pair_sqnorm"], r.topk_w,
                                          r.expert_offsets, r.sorted_pair_ids, self.E, out_dtype, y=b["y"],
                                          saliency=b["saliency"])
        else:
            ops.moe_combine(b["pair_out"], b["pair_scale"], T, self.k, out_dtype, y=b["y"])
        mark(4)
        return LayerOut(b["y"], r, b["x_codes"], b["x_scales"], b["pair_out"], b["pair_scale"], b["pair_sqnorm"], sal,
                        b.get("shared_out"), b["h_codes"], b["h_scales"])

    __call__ = forward
