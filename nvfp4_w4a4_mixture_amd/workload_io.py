"""Materialize the seeded synthetic workloads on the GPU.

Used by bench.py, the GPU tests and the smoke check: draws the BF16 inputs
from ``workloads.gen`` on the host, copies them to device memory, and builds
an :class:`NVFP4MoELayer` whose expert weights are quantized by the library's
own ``nvfp4_quantize_weights`` (offline RTN, per expert Linear).
"""

from __future__ import annotations

import numpy as np
import torch

from workloads import gen
from workloads.configs import LayerConfig, WeightSet

from .layer import NVFP4MoELayer


def bf16_to_device(bits: np.ndarray, device) -> torch.Tensor:
    """uint16 BF16 bit patterns -> torch.bfloat16 tensor on `device`."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def expert_weights_bf16(ws: WeightSet, device, threads: int | None = None):
    """w13 [E, 2I, H] (gate rows, then up rows) and w2 [E, H, I] BF16 on `device`."""
    w13 = torch.empty((ws.E, 2 * ws.I, ws.H), dtype=torch.bfloat16, device=device)
    w2 = torch.empty((ws.E, ws.H, ws.I), dtype=torch.bfloat16, device=device)
    for e, g, u, d in gen.iter_experts_bf16(ws, threads=threads):
        w13[e, : ws.I] = bf16_to_device(g, device)
        w13[e, ws.I:] = bf16_to_device(u, device)
        w2[e] = bf16_to_device(d, device)
    return w13, w2


def build_layer(cfg: LayerConfig, device="cuda", threads: int | None = None,
                keep_bf16: bool = False) -> tuple[NVFP4MoELayer, dict]:
    ws = cfg.weights
    w13, w2 = expert_weights_bf16(ws, device, threads)
    gs_x, gs_h = gen.global_scales(ws)
    layer = NVFP4MoELayer.from_bf16(
        bf16_to_device(gen.router_weight(ws), device),
        torch.from_numpy(gen.router_bias(cfg)).to(device),
        cfg.k, cfg.rsf,
        torch.tensor([gs_x], dtype=torch.float32, device=device),
        torch.from_numpy(gs_h).to(device),
        w13, w2)
    extra = {}
    if keep_bf16:
        extra = {"w13_bf16": w13, "w2_bf16": w2}
    else:
        del w13, w2
    torch.cuda.synchronize()
    return layer, extra


def shared_expert(ws: WeightSet, device="cuda") -> tuple[torch.Tensor, torch.Tensor]:
    """The BF16 shared expert of a weight set: w13 [2I, H] (gate rows, then up rows), w2 [H, I]."""
    g, u, d = gen.shared_expert_bf16(ws)
    return bf16_to_device(np.concatenate([g, u], axis=0), device), bf16_to_device(d, device)


def tokens(cfg: LayerConfig, device="cuda", T: int | None = None) -> torch.Tensor:
    return bf16_to_device(gen.tokens(cfg, T), device)
