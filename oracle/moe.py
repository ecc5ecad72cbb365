"""Routed-expert SwiGLU FFN with NVFP4 W4A4, weighted combine, REAP saliency (oracle).

What the pages fix:

* "K-EXAONE-152B-A23B-REAP-80E-NVFP4" model card, section "Quantization
  Setup": every routed expert Linear is NVFP4 W4A4 -- FP4 weights with their
  own scales per expert Linear module, and the Linear's input activation
  quantized dynamically to FP4 against a calibrated global scale
  (``QuantizationModifier(targets="Linear", scheme="NVFP4")`` covers the
  gate, up and down projections alike); calibration observes the activation
  global scales.
* "K-EXAONE-152B-A23B-REAP-80E-BF16" model card, section "Pruning Setup":
  the routing weights are the renormalized sigmoid weights including
  ``routed_scaling_factor``, and the REAP saliency of expert e is
  mean(topk_weight * ||f_e(x)||_2) over the tokens routed to e.

Readings (pages silent):

* the expert is SwiGLU: h = silu(x W_gate^T) * (x W_up^T), f = h W_down^T, with
  the gate rows stored before the up rows in the fused gate_up weight;
* each matmul is exact float64 over the dequantized operands;
* h is rounded once to float32 and re-quantized from float32 with the expert's
  calibrated global scale gs_h[e] (no BF16 round trip);
* the layer output is y_t = sum_j w_{t,j} f_{e_{t,j}}(x_t) in float64;
* REAP uses the unweighted f and the routing weight w (which includes rsf);
  an expert with no routed pairs has saliency 0;
* calibration: gs_x = 2688 / amax(x_cal); gs_h[e] = 2688 / amax(h_e(x_cal)),
  every calibration token passed densely through every expert.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Sequence

import numpy as np

from . import nvfp4, routing


@dataclass
class ExpertQ:
    """One expert's NVFP4 weights in the canonical layout (packed codes, low nibble first).

    gate/up: [I, H/2] codes, [I, H/16] scales; down: [H, I/2] codes, [H, I/16] scales.
    """

    gate_codes: np.ndarray
    gate_scales: np.ndarray
    gate_gs: np.float32
    up_codes: np.ndarray
    up_scales: np.ndarray
    up_gs: np.float32
    down_codes: np.ndarray
    down_scales: np.ndarray
    down_gs: np.float32

    def dequantized(self):
        """(W_gate [I,H], W_up [I,H], W_down [H,I]) as float64."""
        return (
            nvfp4.dequantize_packed(self.gate_codes, self.gate_scales, self.gate_gs),
            nvfp4.dequantize_packed(self.up_codes, self.up_scales, self.up_gs),
            nvfp4.dequantize_packed(self.down_codes, self.down_scales, self.down_gs),
        )


def quantize_expert(w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> ExpertQ:
    """Offline RTN of one expert's three Linear weights (float32 values of BF16 weights)."""
    gc, gsc, ggs = nvfp4.quantize_weight(w_gate)
    uc, usc, ugs = nvfp4.quantize_weight(w_up)
    dc, dsc, dgs = nvfp4.quantize_weight(w_down)
    return ExpertQ(gc, gsc, ggs, uc, usc, ugs, dc, dsc, dgs)


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def expert_hidden(xhat: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray) -> np.ndarray:
    """h = f32(silu(xhat W_gate^T) * (xhat W_up^T)); matmuls in float64, one rounding to f32."""
    g = xhat @ w_gate.T
    u = xhat @ w_up.T
    return (silu(g) * u).astype(np.float32)


def expert_ffn(xhat: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray,
               gs_h) -> tuple[np.ndarray, np.ndarray]:
    """One expert on dequantized input rows xhat [M, H].

    Returns ``(f [M, H] float64, h [M, I] float32)``: h is quantized with gs_h,
    dequantized, and multiplied by the dequantized down weight.
    """
    h = expert_hidden(xhat, w_gate, w_up)
    hc, hs = nvfp4.quantize(h, gs_h)
    hhat = nvfp4.dequantize(hc, hs, gs_h)
    return hhat @ w_down.T, h


def reap_saliency(pair_f_norm: np.ndarray, weights: np.ndarray, ids: np.ndarray, E: int) -> np.ndarray:
    """S_e = (sum over pairs p routed to e of w_p * ||f_p||_2) / count_e; 0 if count_e == 0."""
    ids = np.asarray(ids).reshape(-1)
    wn = np.asarray(weights, dtype=np.float64).reshape(-1) * np.asarray(pair_f_norm, dtype=np.float64).reshape(-1)
    num = np.zeros(E, dtype=np.float64)
    np.add.at(num, ids, wn)
    cnt = np.bincount(ids, minlength=E)
    out = np.zeros(E, dtype=np.float64)
    nz = cnt > 0
    out[nz] = num[nz] / cnt[nz]
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of BF16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


ExpertSource = Callable[[int], ExpertQ]


def _expert_getter(experts) -> ExpertSource:
    if callable(experts):
        return experts
    return lambda e: experts[e]


def moe_layer(x_bf16: np.ndarray, w_router_bf16: np.ndarray, bias: np.ndarray, k: int, rsf: float,
              gs_x, experts, gs_h: np.ndarray, tokens: Sequence[int] | None = None,
              with_pairs: bool = False, threads: int = 1) -> dict:
    """The routed MoE layer, end to end, on the CPU.

    ``experts`` is a sequence of :class:`ExpertQ` or a callable e -> ExpertQ
    (so large configurations can produce experts lazily).  ``tokens`` restricts
    the computation to a subset of token rows (routing and quantization are
    per token, so each selected row is computed exactly as in the full layer).

    Returns a dict with ``ids``, ``weights`` (float32), ``weights64``, ``gap``,
    ``x_codes`` / ``x_scales`` (unpacked codes, E4M3 bytes), ``y`` (float64
    [len(tokens), H]) and, over the routed experts, ``saliency`` (float64 [E],
    only meaningful when ``tokens`` is None), ``pair_norm`` (||f_p||_2 per pair)
    and, if ``with_pairs``, ``pair_f`` (unweighted f per pair, [n*k, H]).
    ``threads`` > 1 evaluates the experts concurrently; their contributions are
    still added to y one expert after another in increasing expert order, so
    the result does not depend on it.
    """
    get = _expert_getter(experts)
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    if tokens is not None:
        x_bf16 = x_bf16[np.asarray(tokens, dtype=np.int64)]
    n, H = x_bf16.shape
    E = w_router_bf16.shape[0]
    ids, w32, w64, gap = routing.route(x_bf16, w_router_bf16, bias, k, rsf)
    xc, xs = nvfp4.quantize(bf16_to_f32(x_bf16), gs_x)
    xhat = nvfp4.dequantize(xc, xs, gs_x)

    pair_norm = np.zeros(n * k, dtype=np.float64)
    pair_f = np.zeros((n * k, H), dtype=np.float64) if with_pairs else None
    y = np.zeros((n, H), dtype=np.float64)
    flat = ids.reshape(-1)

    def one(e):
        pairs = np.nonzero(flat == e)[0]
        wg, wu, wd = get(int(e)).dequantized()
        f, _ = expert_ffn(xhat[pairs // k], wg, wu, wd, gs_h[e])
        return pairs, f

    routed = [int(e) for e in np.unique(flat)]
    if threads > 1:
        from concurrent.futures import ThreadPoolExecutor
        ex = ThreadPoolExecutor(threads)
        results = ex.map(one, routed)  # yields in expert order
    else:
        ex = None
        results = map(one, routed)
    for pairs, f in results:
        toks = pairs // k
        pair_norm[pairs] = np.sqrt(np.sum(f * f, axis=1))
        if with_pairs:
            pair_f[pairs] = f
        # y_t += w_{t,j} f_p  (each pair appears once; order of j does not matter in fp64)
        np.add.at(y, toks, w64.reshape(-1)[pairs][:, None] * f)
    if ex is not None:
        ex.shutdown()
    sal = reap_saliency(pair_norm, w64, ids, E)
    return dict(ids=ids, weights=w32, weights64=w64, gap=gap, x_codes=xc, x_scales=xs, y=y,
                saliency=sal, pair_norm=pair_norm, pair_f=pair_f)


def expert_pairs_output(x_bf16_rows: np.ndarray, gs_x, expert: ExpertQ, gs_h_e) -> np.ndarray:
    """Unweighted f [M, H] of the given token rows through one expert, as the layer computes it.

    Each row is quantized to NVFP4 with gs_x and dequantized (quantization is
    per row, so the subset gives the same values as the whole batch), then
    passed through :func:`expert_ffn` with the expert's calibrated gs_h."""
    xc, xs = nvfp4.quantize(bf16_to_f32(x_bf16_rows), gs_x)
    xhat = nvfp4.dequantize(xc, xs, gs_x)
    wg, wu, wd = expert.dequantized()
    f, _ = expert_ffn(xhat, wg, wu, wd, gs_h_e)
    return f


def calibrate(x_cal_bf16: np.ndarray, experts, E: int, threads: int = 1) -> tuple[np.float32, np.ndarray]:
    """Static global scales from a calibration batch: (gs_x, gs_h [E] float32).

    gs_x = 2688 / amax(x_cal); gs_h[e] = 2688 / amax(h_e) with every calibration
    token passed through every expert (dense), h computed as in the layer.
    ``threads`` > 1 evaluates experts concurrently (results do not depend on it).
    """
    get = _expert_getter(experts)
    xf = bf16_to_f32(x_cal_bf16)
    gs_x = nvfp4.global_scale(np.max(np.abs(xf)))
    xc, xs = nvfp4.quantize(xf, gs_x)
    xhat = nvfp4.dequantize(xc, xs, gs_x)

    def one(e):
        wg, wu, _ = get(e).dequantized()
        h = expert_hidden(xhat, wg, wu)
        return nvfp4.global_scale(np.max(np.abs(h)))

    if threads > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(threads) as ex:
            vals = list(ex.map(one, range(E)))
    else:
        vals = [one(e) for e in range(E)]
    return gs_x, np.array(vals, dtype=np.float32)
