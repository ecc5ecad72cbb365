"""Python binding of the C ABI, one function per entry point, same names.

Argument marshalling only: each function checks tensor shapes/dtypes/devices,
allocates missing outputs with torch (device memory), passes raw pointers and
the current HIP stream to the library, and raises :class:`MoEError` on a
non-OK status.  Every step of the layer runs in the library's HIP kernels.
"""

from __future__ import annotations

import ctypes
from typing import NamedTuple, Optional

import torch

from ._lib import MoEError, check, lib  # noqa: F401

__all__ = ["moe_route", "moe_route_quantize", "nvfp4_quantize_act", "nvfp4_quantize_weights", "moe_nvfp4_grouped_ffn",
           "moe_nvfp4_grouped_ffn_noalloc", "moe_nvfp4_gate_up_swiglu", "moe_nvfp4_down_scatter", "moe_combine", "reap_saliency",
           "moe_combine_reap", "reap_prune_select", "moe_gather_experts", "moe_shared_workspace_bytes", "moe_shared_expert",
           "moe_shared_gate_up", "moe_shared_down", "moe_combine_block", "hadamard_rotate_bf16",
           "moe_nvfp4_prepack_weights", "moe_nvfp4_unpack_weights",
           "moe_route_workspace_bytes", "moe_ffn_workspace_bytes", "moe_ffn_stage_workspace_bytes", "RouteOut"]


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None, contiguous: bool = True) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None:
        return ws
    # torch's caching allocator returns 256-byte aligned blocks
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def moe_route_workspace_bytes(T: int, H: int, E: int, k: int) -> int:
    return int(lib().moe_route_workspace_bytes(T, H, E, k))


def moe_ffn_workspace_bytes(T: int, k: int, E: int, H: int, I: int) -> int:
    return int(lib().moe_ffn_workspace_bytes(T, k, E, H, I))


def moe_ffn_stage_workspace_bytes(T: int, k: int, E: int, H: int, I: int) -> int:
    return int(lib().moe_ffn_stage_workspace_bytes(T, k, E, H, I))


class RouteOut(NamedTuple):
    topk_ids: torch.Tensor  # [T, k] int32
    topk_w: torch.Tensor  # [T, k] float32
    expert_counts: torch.Tensor  # [E] int32
    expert_offsets: torch.Tensor  # [E+1] int32
    sorted_pair_ids: torch.Tensor  # [T*k] int32


def moe_route(x_bf16: torch.Tensor, w_router_bf16: torch.Tensor, bias: torch.Tensor, k: int,
              routed_scaling_factor: float, out: Optional[RouteOut] = None,
              workspace: Optional[torch.Tensor] = None, stream=None) -> RouteOut:
    if x_bf16.dim() != 2 or (x_bf16.numel() > 0 and x_bf16.stride(1) != 1):
        raise ValueError("x_bf16 must be [T, H] with unit column stride")
    _need(x_bf16, "x_bf16", torch.bfloat16, contiguous=False)
    T, H = x_bf16.shape
    ldx = x_bf16.stride(0) if T > 0 else H
    E = w_router_bf16.shape[0]
    _need(w_router_bf16, "w_router_bf16", torch.bfloat16, (E, H))
    _need(bias, "bias", torch.float32, (E,))
    dev = x_bf16.device
    if out is None:
        out = RouteOut(torch.empty((T, k), dtype=torch.int32, device=dev),
                       torch.empty((T, k), dtype=torch.float32, device=dev),
                       torch.empty((E,), dtype=torch.int32, device=dev),
                       torch.empty((E + 1,), dtype=torch.int32, device=dev),
                       torch.empty((T * k,), dtype=torch.int32, device=dev))
    nbytes = moe_route_workspace_bytes(T, H, E, k)
    ws = _workspace(nbytes, dev, workspace)
    st = lib().moe_route(_p(x_bf16), T, H, ldx, _p(w_router_bf16), _p(bias), E, k,
                         float(routed_scaling_factor), _p(out.topk_ids), _p(out.topk_w), _p(out.expert_counts),
                         _p(out.expert_offsets), _p(out.sorted_pair_ids), _p(ws), ws.numel(), _stream(stream))
    check(st, "moe_route")
    return out


def moe_route_quantize(x_bf16: torch.Tensor, w_router_bf16: torch.Tensor, bias: torch.Tensor, k: int,
                       routed_scaling_factor: float, x_gs: torch.Tensor, out: Optional[RouteOut] = None,
                       x_codes: Optional[torch.Tensor] = None, x_scales: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None):
    """moe_route plus the NVFP4 quantization of x in the same pass: (RouteOut, x_codes, x_scales)."""
    if x_bf16.dim() != 2 or (x_bf16.numel() > 0 and x_bf16.stride(1) != 1):
        raise ValueError("x_bf16 must be [T, H] with unit column stride")
    _need(x_bf16, "x_bf16", torch.bfloat16, contiguous=False)
    T, H = x_bf16.shape
    ldx = x_bf16.stride(0) if T > 0 else H
    E = w_router_bf16.shape[0]
    _need(w_router_bf16, "w_router_bf16", torch.bfloat16, (E, H))
    _need(bias, "bias", torch.float32, (E,))
    _need(x_gs, "x_gs", torch.float32, (1,))
    dev = x_bf16.device
    if out is None:
        out = RouteOut(torch.empty((T, k), dtype=torch.int32, device=dev),
                       torch.empty((T, k), dtype=torch.float32, device=dev),
                       torch.empty((E,), dtype=torch.int32, device=dev),
                       torch.empty((E + 1,), dtype=torch.int32, device=dev),
                       torch.empty((T * k,), dtype=torch.int32, device=dev))
    if x_codes is None:
        x_codes = torch.empty((T, H // 2), dtype=torch.uint8, device=dev)
    if x_scales is None:
        x_scales = torch.empty((T, H // 16), dtype=torch.uint8, device=dev)
    _need(x_codes, "x_codes", torch.uint8, (T, H // 2))
    _need(x_scales, "x_scales", torch.uint8, (T, H // 16))
    nbytes = moe_route_workspace_bytes(T, H, E, k)
    ws = _workspace(nbytes, dev, workspace)
    st = lib().moe_route_quantize(_p(x_bf16), T, H, ldx, _p(w_router_bf16), _p(bias), E, k,
                                  float(routed_scaling_factor), _p(x_gs), _p(x_codes), _p(x_scales),
                                  _p(out.topk_ids), _p(out.topk_w), _p(out.expert_counts), _p(out.expert_offsets),
                                  _p(out.sorted_pair_ids), _p(ws), ws.numel(), _stream(stream))
    check(st, "moe_route_quantize")
    return out, x_codes, x_scales


def nvfp4_quantize_act(x_bf16: torch.Tensor, global_scale: torch.Tensor, codes: Optional[torch.Tensor] = None,
                       scales: Optional[torch.Tensor] = None, stream=None):
    if x_bf16.dim() != 2 or (x_bf16.numel() > 0 and x_bf16.stride(1) != 1):
        raise ValueError("x_bf16 must be [rows, cols] with unit column stride")
    _need(x_bf16, "x_bf16", torch.bfloat16, contiguous=False)
    _need(global_scale, "global_scale", torch.float32, (1,))
    rows, cols = x_bf16.shape
    ld = x_bf16.stride(0) if rows > 0 else cols
    dev = x_bf16.device
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
    st = lib().nvfp4_quantize_act(_p(x_bf16), rows, cols, ld, _p(global_scale), _p(codes),
                                  _p(scales), _stream(stream))
    check(st, "nvfp4_quantize_act")
    return codes, scales


def nvfp4_quantize_weights(w_bf16: torch.Tensor, stream=None):
    """w_bf16 [batch, rows, cols] -> (codes [batch, rows, cols/2], scales, gs [batch]).

    scales are in the tiled weight layout, shaped [batch, rows/16, cols/128, 16, 8]:
    scales[b, i, j, r, q] is the scale of row 16 i + r, columns 128 j + 16 q .. + 15."""
    _need(w_bf16, "w_bf16", torch.bfloat16)
    if w_bf16.dim() != 3:
        raise ValueError("w_bf16 must be [batch, rows, cols]")
    b, r, c = w_bf16.shape
    dev = w_bf16.device
    codes = torch.empty((b, r, c // 2), dtype=torch.uint8, device=dev)
    if r % 16 or c % 128:
        raise ValueError("nvfp4_quantize_weights needs rows % 16 == 0 and cols % 128 == 0")
    scales = torch.empty((b, r // 16, c // 128, 16, 8), dtype=torch.uint8, device=dev)
    gs = torch.empty((b,), dtype=torch.float32, device=dev)
    st = lib().nvfp4_quantize_weights(_p(w_bf16), b, r, c, _p(codes), _p(scales), _p(gs), _stream(stream))
    check(st, "nvfp4_quantize_weights")
    return codes, scales, gs


def _ffn_dims(x_codes, w13_codes, w2_codes):
    T = x_codes.shape[0]
    E, two_i, h_half = w13_codes.shape
    return T, 2 * h_half, E, two_i // 2


def _pair_outputs(npairs: int, H: int, dev, pair_out, pair_scale, pair_sqnorm):
    """The pair-row outputs: given ones checked, missing ones allocated (pair_sqnorm True: allocate, None/False: skip)."""
    if pair_out is None:
        pair_out = torch.empty((npairs, H), dtype=torch.float16, device=dev)
    if pair_scale is None:
        pair_scale = torch.empty((npairs,), dtype=torch.float32, device=dev)
    _need(pair_out, "pair_out", torch.float16, (npairs, H))
    _need(pair_scale, "pair_scale", torch.float32, (npairs,))
    if pair_sqnorm is True:
        pair_sqnorm = torch.empty((npairs,), dtype=torch.float32, device=dev)
    elif pair_sqnorm is False:
        pair_sqnorm = None
    if pair_sqnorm is not None:
        _need(pair_sqnorm, "pair_sqnorm", torch.float32, (npairs,))
    return pair_out, pair_scale, pair_sqnorm


def moe_nvfp4_grouped_ffn(x_codes, x_scales, x_gs, w13_codes, w13_scales, w13_gs, w2_codes, w2_scales, w2_gs,
                          h_gs, k: int, expert_offsets, sorted_pair_ids, topk_w, pair_out=None, pair_scale=None,
                          pair_sqnorm: Optional[torch.Tensor] | bool = None, workspace=None, stream=None):
    """Returns (pair_out, pair_scale, pair_sqnorm): pair row p is pair_out[p] (FP16) * pair_scale[p]."""
    T, H, E, I = _ffn_dims(x_codes, w13_codes, w2_codes)
    _need(x_codes, "x_codes", torch.uint8, (T, H // 2))
    _need(x_scales, "x_scales", torch.uint8, (T, H // 16))
    _need(x_gs, "x_gs", torch.float32, (1,))
    _need(w13_codes, "w13_codes", torch.uint8, (E, 2 * I, H // 2))
    _need(w13_scales, "w13_scales", torch.uint8, (E, 2 * I // 16, H // 128, 16, 8))
    _need(w13_gs, "w13_gs", torch.float32, (E, 2))
    _need(w2_codes, "w2_codes", torch.uint8, (E, H, I // 2))
    _need(w2_scales, "w2_scales", torch.uint8, (E, H // 16, I // 128, 16, 8))
    _need(w2_gs, "w2_gs", torch.float32, (E,))
    _need(h_gs, "h_gs", torch.float32, (E,))
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    _need(sorted_pair_ids, "sorted_pair_ids", torch.int32, (T * k,))
    _need(topk_w, "topk_w", torch.float32)
    dev = x_codes.device
    pair_out, pair_scale, pair_sqnorm = _pair_outputs(T * k, H, dev, pair_out, pair_scale, pair_sqnorm)
    ws = _workspace(moe_ffn_workspace_bytes(T, k, E, H, I), dev, workspace)
    st = lib().moe_nvfp4_grouped_ffn(_p(x_codes), _p(x_scales), _p(x_gs), T, H, _p(w13_codes), _p(w13_scales),
                                     _p(w13_gs), _p(w2_codes), _p(w2_scales), _p(w2_gs), _p(h_gs), E, I, k,
                                     _p(expert_offsets), _p(sorted_pair_ids), _p(topk_w), _p(pair_out),
                                     _p(pair_scale), _p(pair_sqnorm), _p(ws), ws.numel(), _stream(stream))
    check(st, "moe_nvfp4_grouped_ffn")
    return pair_out, pair_scale, pair_sqnorm


def moe_nvfp4_grouped_ffn_noalloc(x_codes, x_scales, x_gs, w13_codes, w13_scales, w13_gs, w2_codes, w2_scales,
                                  w2_gs, h_gs, k: int, expert_offsets, sorted_pair_ids, topk_w, pair_out, pair_scale,
                                  pair_sqnorm: Optional[torch.Tensor] = None, stream=None):
    """moe_nvfp4_grouped_ffn on the library's static scratch: the caller passes every output
    (nothing is allocated here or in the library, so the call can be captured in a graph)."""
    T, H, E, I = _ffn_dims(x_codes, w13_codes, w2_codes)
    _need(x_codes, "x_codes", torch.uint8, (T, H // 2))
    _need(x_scales, "x_scales", torch.uint8, (T, H // 16))
    _need(x_gs, "x_gs", torch.float32, (1,))
    _need(w13_codes, "w13_codes", torch.uint8, (E, 2 * I, H // 2))
    _need(w13_scales, "w13_scales", torch.uint8, (E, 2 * I // 16, H // 128, 16, 8))
    _need(w13_gs, "w13_gs", torch.float32, (E, 2))
    _need(w2_codes, "w2_codes", torch.uint8, (E, H, I // 2))
    _need(w2_scales, "w2_scales", torch.uint8, (E, H // 16, I // 128, 16, 8))
    _need(w2_gs, "w2_gs", torch.float32, (E,))
    _need(h_gs, "h_gs", torch.float32, (E,))
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    _need(sorted_pair_ids, "sorted_pair_ids", torch.int32, (T * k,))
    _need(topk_w, "topk_w", torch.float32)
    _need(pair_out, "pair_out", torch.float16, (T * k, H))
    _need(pair_scale, "pair_scale", torch.float32, (T * k,))
    if pair_sqnorm is not None:
        _need(pair_sqnorm, "pair_sqnorm", torch.float32, (T * k,))
    st = lib().moe_nvfp4_grouped_ffn_noalloc(_p(x_codes), _p(x_scales), _p(x_gs), T, H, _p(w13_codes),
                                             _p(w13_scales), _p(w13_gs), _p(w2_codes), _p(w2_scales), _p(w2_gs),
                                             _p(h_gs), E, I, k, _p(expert_offsets), _p(sorted_pair_ids), _p(topk_w),
                                             _p(pair_out), _p(pair_scale), _p(pair_sqnorm), _stream(stream))
    check(st, "moe_nvfp4_grouped_ffn_noalloc")
    return pair_out, pair_scale, pair_sqnorm


def moe_nvfp4_gate_up_swiglu(x_codes, x_scales, x_gs, w13_codes, w13_scales, w13_gs, h_gs, k: int,
                             expert_offsets, sorted_pair_ids, h_codes=None, h_scales=None, workspace=None,
                             stream=None):
    T = x_codes.shape[0]
    E, two_i, h_half = w13_codes.shape
    H, I = 2 * h_half, two_i // 2
    _need(x_codes, "x_codes", torch.uint8, (T, H // 2))
    _need(w13_scales, "w13_scales", torch.uint8, (E, 2 * I // 16, H // 128, 16, 8))
    dev = x_codes.device
    if h_codes is None:
        h_codes = torch.empty((T * k, I // 2), dtype=torch.uint8, device=dev)
    if h_scales is None:
        h_scales = torch.empty((T * k, I // 16), dtype=torch.uint8, device=dev)
    ws = _workspace(moe_ffn_stage_workspace_bytes(T, k, E, H, I), dev, workspace)
    st = lib().moe_nvfp4_gate_up_swiglu(_p(x_codes), _p(x_scales), _p(x_gs), T, H, _p(w13_codes), _p(w13_scales),
                                        _p(w13_gs), _p(h_gs), E, I, k, _p(expert_offsets), _p(sorted_pair_ids),
                                        _p(h_codes), _p(h_scales), _p(ws), ws.numel(), _stream(stream))
    check(st, "moe_nvfp4_gate_up_swiglu")
    return h_codes, h_scales


def moe_nvfp4_down_scatter(h_codes, h_scales, h_gs, T: int, w2_codes, w2_scales, w2_gs, k: int, expert_offsets,
                           sorted_pair_ids, topk_w, pair_out=None, pair_scale=None, pair_sqnorm=None, workspace=None,
                           stream=None):
    """Returns (pair_out, pair_scale, pair_sqnorm), as moe_nvfp4_grouped_ffn."""
    E, H, i_half = w2_codes.shape
    I = 2 * i_half
    _need(h_codes, "h_codes", torch.uint8, (T * k, I // 2))
    dev = h_codes.device
    pair_out, pair_scale, pair_sqnorm = _pair_outputs(T * k, H, dev, pair_out, pair_scale, pair_sqnorm)
    ws = _workspace(moe_ffn_stage_workspace_bytes(T, k, E, H, I), dev, workspace)
    st = lib().moe_nvfp4_down_scatter(_p(h_codes), _p(h_scales), _p(h_gs), T, H, _p(w2_codes), _p(w2_scales),
                                      _p(w2_gs), E, I, k, _p(expert_offsets), _p(sorted_pair_ids), _p(topk_w),
                                      _p(pair_out), _p(pair_scale), _p(pair_sqnorm), _p(ws), ws.numel(),
                                      _stream(stream))
    check(st, "moe_nvfp4_down_scatter")
    return pair_out, pair_scale, pair_sqnorm


def _need_pairs(pair_out: torch.Tensor, pair_scale: torch.Tensor, T: int, k: int) -> int:
    _need(pair_out, "pair_out", torch.float16)
    if pair_out.dim() != 2 or pair_out.shape[0] < T * k:
        raise ValueError(f"pair_out must be [>= T*k, H], got {tuple(pair_out.shape)}")
    _need(pair_scale, "pair_scale", torch.float32)
    if pair_scale.numel() < T * k:
        raise ValueError(f"pair_scale must hold T*k = {T * k} scales, got {pair_scale.numel()}")
    return pair_out.shape[1]


def moe_combine(pair_out: torch.Tensor, pair_scale: torch.Tensor, T: int, k: int,
                out_dtype: torch.dtype = torch.bfloat16, y=None, stream=None) -> torch.Tensor:
    H = _need_pairs(pair_out, pair_scale, T, k)
    code = {torch.bfloat16: 0, torch.float32: 1}[out_dtype]
    if y is None:
        y = torch.empty((T, H), dtype=out_dtype, device=pair_out.device)
    st = lib().moe_combine(_p(pair_out), _p(pair_scale), T, k, H, code, _p(y), _stream(stream))
    check(st, "moe_combine")
    return y


def moe_combine_reap(pair_out: torch.Tensor, pair_scale: torch.Tensor, T: int, k: int, pair_sqnorm, topk_w,
                     expert_offsets, sorted_pair_ids, E: int, out_dtype: torch.dtype = torch.bfloat16, y=None,
                     saliency=None, stream=None):
    """moe_combine and reap_saliency in one launch: (y, saliency)."""
    H = _need_pairs(pair_out, pair_scale, T, k)
    code = {torch.bfloat16: 0, torch.float32: 1}[out_dtype]
    if y is None:
        y = torch.empty((T, H), dtype=out_dtype, device=pair_out.device)
    if saliency is None:
        saliency = torch.empty((E,), dtype=torch.float32, device=pair_out.device)
    st = lib().moe_combine_reap(_p(pair_out), _p(pair_scale), T, k, H, code, _p(y), _p(pair_sqnorm), _p(topk_w),
                                _p(expert_offsets), _p(sorted_pair_ids), E, _p(saliency), _stream(stream))
    check(st, "moe_combine_reap")
    return y, saliency


def reap_saliency(pair_sqnorm, topk_w, expert_offsets, sorted_pair_ids, T: int, k: int, E: int, out=None,
                  stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty((E,), dtype=torch.float32, device=pair_sqnorm.device)
    st = lib().reap_saliency(_p(pair_sqnorm), _p(topk_w), _p(expert_offsets), _p(sorted_pair_ids), T, k, E,
                             _p(out), _stream(stream))
    check(st, "reap_saliency")
    return out


def reap_prune_select(saliency: torch.Tensor, n_keep: int, out=None, stream=None) -> torch.Tensor:
    """INT32 ids of the n_keep highest-saliency experts, ascending."""
    _need(saliency, "saliency", torch.float32)
    E = saliency.shape[0]
    if out is None:
        out = torch.empty((n_keep,), dtype=torch.int32, device=saliency.device)
    _need(out, "keep_ids", torch.int32, (n_keep,))
    st = lib().reap_prune_select(_p(saliency), E, n_keep, _p(out), _stream(stream))
    check(st, "reap_prune_select")
    return out


def moe_gather_experts(src: torch.Tensor, keep_ids: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """out[i] = src[keep_ids[i]] for a per-expert tensor src [E, ...] (any dtype)."""
    if not isinstance(src, torch.Tensor) or src.device.type != "cuda" or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    _need(keep_ids, "keep_ids", torch.int32)
    n = keep_ids.shape[0]
    if out is None:
        out = torch.empty((n, *src.shape[1:]), dtype=src.dtype, device=src.device)
    _need(out, "out", src.dtype, (n, *src.shape[1:]))
    per = src[0].numel() * src.element_size() if src.shape[0] > 0 else 0
    st = lib().moe_gather_experts(_p(src), src.shape[0], per, _p(keep_ids), n, _p(out), _stream(stream))
    check(st, "moe_gather_experts")
    return out


def moe_shared_workspace_bytes(T: int, H: int, I: int) -> int:
    return int(lib().moe_shared_workspace_bytes(T, H, I))


def _shared_dims(x_bf16, w13_bf16, w2_bf16):
    if x_bf16.dim() != 2 or x_bf16.stride(1) != 1:
        raise ValueError("x_bf16 must be [T, H] with unit column stride")
    T, H = x_bf16.shape
    _need(w13_bf16, "w13_bf16", torch.bfloat16)
    I = w13_bf16.shape[0] // 2
    _need(w13_bf16, "w13_bf16", torch.bfloat16, (2 * I, H))
    _need(w2_bf16, "w2_bf16", torch.bfloat16, (H, I))
    return T, H, I


def moe_shared_expert(x_bf16, w13_bf16, w2_bf16, out=None, workspace=None, stream=None) -> torch.Tensor:
    """BF16 shared expert: FP32 [T, H] = bf16(silu(x Wg^T) * (x Wu^T)) . Wd^T."""
    _need(x_bf16, "x_bf16", torch.bfloat16, contiguous=False)
    T, H, I = _shared_dims(x_bf16, w13_bf16, w2_bf16)
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x_bf16.device)
    _need(out, "shared_out", torch.float32, (T, H))
    nb = moe_shared_workspace_bytes(T, H, I)
    ws = _workspace(nb, x_bf16.device, workspace)
    st = lib().moe_shared_expert(_p(x_bf16), T, H, x_bf16.stride(0), _p(w13_bf16), _p(w2_bf16), I, _p(out), _p(ws),
                                 ws.numel(), _stream(stream))
    check(st, "moe_shared_expert")
    return out


def moe_shared_gate_up(x_bf16, w13_bf16, h=None, workspace=None, stream=None) -> torch.Tensor:
    _need(x_bf16, "x_bf16", torch.bfloat16, contiguous=False)
    if x_bf16.dim() != 2 or x_bf16.stride(1) != 1:
        raise ValueError("x_bf16 must be [T, H] with unit column stride")
    T, H = x_bf16.shape
    _need(w13_bf16, "w13_bf16", torch.bfloat16)
    I = w13_bf16.shape[0] // 2
    _need(w13_bf16, "w13_bf16", torch.bfloat16, (2 * I, H))
    if h is None:
        h = torch.empty((T, I), dtype=torch.bfloat16, device=x_bf16.device)
    _need(h, "h_bf16", torch.bfloat16, (T, I))
    ws = _workspace(moe_shared_workspace_bytes(T, H, I), x_bf16.device, workspace)
    st = lib().moe_shared_gate_up(_p(x_bf16), T, H, x_bf16.stride(0), _p(w13_bf16), I, _p(h), _p(ws), ws.numel(),
                                  _stream(stream))
    check(st, "moe_shared_gate_up")
    return h


def moe_shared_down(h_bf16, w2_bf16, out=None, workspace=None, stream=None) -> torch.Tensor:
    _need(h_bf16, "h_bf16", torch.bfloat16)
    T, I = h_bf16.shape
    _need(w2_bf16, "w2_bf16", torch.bfloat16)
    H = w2_bf16.shape[0]
    _need(w2_bf16, "w2_bf16", torch.bfloat16, (H, I))
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=h_bf16.device)
    _need(out, "shared_out", torch.float32, (T, H))
    ws = _workspace(moe_shared_workspace_bytes(T, H, I), h_bf16.device, workspace)
    st = lib().moe_shared_down(_p(h_bf16), T, I, _p(w2_bf16), H, _p(out), _p(ws), ws.numel(), _stream(stream))
    check(st, "moe_shared_down")
    return out


def moe_combine_block(pair_out: torch.Tensor, pair_scale: torch.Tensor, shared_out: torch.Tensor, T: int, k: int,
                      out_dtype: torch.dtype = torch.bfloat16, y=None, stream=None) -> torch.Tensor:
    """y = routed combine + shared expert output."""
    H = _need_pairs(pair_out, pair_scale, T, k)
    _need(shared_out, "shared_out", torch.float32, (T, H))
    code = {torch.bfloat16: 0, torch.float32: 1}[out_dtype]
    if y is None:
        y = torch.empty((T, H), dtype=out_dtype, device=pair_out.device)
    st = lib().moe_combine_block(_p(pair_out), _p(pair_scale), _p(shared_out), T, k, H, code, _p(y), _stream(stream))
    check(st, "moe_combine_block")
    return y


def hadamard_rotate_bf16(src: torch.Tensor, signs: Optional[torch.Tensor], block: int, out=None,
                         stream=None) -> torch.Tensor:
    """Rows of src [..., cols] (BF16) times D blockdiag(H_block) / sqrt(block); out may be src (in place)."""
    _need(src, "src", torch.bfloat16, contiguous=False)
    if src.stride(-1) != 1:
        raise ValueError("src must have unit column stride")
    cols = src.shape[-1]
    s2 = src.reshape(-1, cols) if src.dim() != 2 else src
    if out is None:
        out = torch.empty(src.shape, dtype=torch.bfloat16, device=src.device)
    _need(out, "out", torch.bfloat16, tuple(src.shape), contiguous=False)
    o2 = out.reshape(-1, cols) if out.dim() != 2 else out
    if o2.data_ptr() != out.data_ptr() or (out.dim() != 2 and not out.is_contiguous()):
        raise ValueError("out must be 2-D or contiguous")
    if signs is not None:
        _need(signs, "signs", torch.float32, (cols,))
    st = lib().hadamard_rotate_bf16(_p(s2), s2.shape[0], cols, s2.stride(0), _p(signs), block, _p(o2), o2.stride(0),
                                    _stream(stream))
    check(st, "hadamard_rotate_bf16")
    return out


def _relayout(fn: str, codes: torch.Tensor, scales: torch.Tensor, kind: int, to_tiled: bool, stream=None):
    _need(codes, "codes", torch.uint8)
    _need(scales, "scales", torch.uint8)
    E, N, kh = codes.shape
    K = 2 * kh
    if to_tiled:
        _need(scales, "scales", torch.uint8, (E, N, K // 16))
        out_s = torch.empty((E, N // 16, K // 128, 16, 8), dtype=torch.uint8, device=codes.device)
    else:
        _need(scales, "scales", torch.uint8, (E, N // 16, K // 128, 16, 8))
        out_s = torch.empty((E, N, K // 16), dtype=torch.uint8, device=codes.device)
    out_c = torch.empty_like(codes)
    st = getattr(lib(), fn)(_p(codes), _p(scales), E, N, K, kind, _p(out_c), _p(out_s), _stream(stream))
    check(st, fn)
    return out_c, out_s


def moe_nvfp4_prepack_weights(codes: torch.Tensor, scales: torch.Tensor, kind: int, stream=None):
    """Canonical (codes [E, N, K/2], scales [E, N, K/16]) -> (codes, tiled scales [E, N/16, K/128, 16, 8])."""
    return _relayout("moe_nvfp4_prepack_weights", codes, scales, kind, True, stream)


def moe_nvfp4_unpack_weights(codes: torch.Tensor, packed_scales: torch.Tensor, kind: int, stream=None):
    """Exact inverse of moe_nvfp4_prepack_weights."""
    return _relayout("moe_nvfp4_unpack_weights", codes, packed_scales, kind, False, stream)
