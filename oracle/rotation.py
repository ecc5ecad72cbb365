"""Offline Hadamard rotation of the hidden dimension before NVFP4 RTN (oracle).

What the pages fix ("[NetsPresso AQ Deep Dive] How to Quantize the
K-EXAONE-236B Model to 4-Bit (NVFP4)", sections on where the outliers sit and
"Offline Fusion of Multiple Quantization Algorithms"): heavy-tail outliers in
a few layers distort the NVFP4 block scale; the remedy rotates the weights'
coordinate system before quantization so that outliers do not pile up in one
block, and the rotation is absorbed into the weights (nothing extra runs at
inference).  The pages name QuaRot among the algorithms combined, and give no
formula; AQ's own transforms are proprietary.

Readings (the plainest rotation of that kind):

* R = D . blockdiag(H_b, ..., H_b) / sqrt(b): D a seeded diagonal of +-1 signs
  over the hidden dimension, H_b the Sylvester Hadamard matrix of a power of
  two b dividing the hidden size (b = hidden size is a full rotation);
* rows are rotated: rot(v) = v R, applied to each token x, to each row of
  W_gate and W_up and to each router row -- so x W^T = rot(x) rot(W)^T exactly,
  and the routing and the expert function are unchanged in exact arithmetic;
  W_down's output side, the residual stream, would carry the inverse rotation
  into the next layer and is left as it is;
* rotated values are rounded once to BF16 (the model's dtype) before the RTN;
  the float64 value rounded is (sum of the +-1 products) / sqrt(b), whose sum is
  exact for BF16 inputs of moderate range;
* the rotated layer calibrates gs_x on the rotated calibration batch and
  reuses gs_h, since h is the same function of x in exact arithmetic.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

from __future__ import annotations

import numpy as np

from . import nvfp4, routing
from .moe import bf16_to_f32, silu
from .shared import round_bf16


def sylvester(b: int) -> np.ndarray:
    """H_b with entries +-1: H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    if b < 1 or b & (b - 1):
        raise ValueError("b must be a power of two")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < b:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate_rows(values: np.ndarray, signs: np.ndarray, b: int) -> np.ndarray:
    """Exact float64 v R for each row v (values [..., n], signs [n] of +-1)."""
    v = np.asarray(values, dtype=np.float64)
    n = v.shape[-1]
    if n % b:
        raise ValueError("b must divide the row length")
    vs = v * np.asarray(signs, dtype=np.float64)
    # the +-1 products are summed first, then divided once by sqrt(b)
    return (vs.reshape(*v.shape[:-1], n // b, b) @ sylvester(b)).reshape(v.shape) / np.sqrt(b)


def rotate_bf16(bits: np.ndarray, signs: np.ndarray, b: int) -> np.ndarray:
    """BF16 bit patterns of bf16(v R) for rows of BF16 bit patterns."""
    r = round_bf16(rotate_rows(bf16_to_f32(bits), signs, b)).astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)  # exact: r holds BF16 values


def moe_layer_reference(x_bf16: np.ndarray, w_router_bf16: np.ndarray, bias: np.ndarray, k: int, rsf: float,
                        experts_bf16, tokens=None) -> dict:
    """The layer without quantization: BF16 inputs and weights, float64 arithmetic.

    ``experts_bf16`` maps e -> (W_gate, W_up, W_down) BF16 bit patterns.  The
    routing is the quantized layer's (it never sees NVFP4 values)."""
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    if tokens is not None:
        x_bf16 = x_bf16[np.asarray(tokens, dtype=np.int64)]
    ids, _, w64, gap = routing.route(x_bf16, w_router_bf16, bias, k, rsf)
    x = bf16_to_f32(x_bf16).astype(np.float64)
    y = np.zeros_like(x)
    flat = ids.reshape(-1)
    for e in np.unique(flat):
        pairs = np.nonzero(flat == e)[0]
        toks = pairs // k
        wg, wu, wd = (bf16_to_f32(a).astype(np.float64) for a in experts_bf16(int(e)))
        xe = x[toks]
        f = (silu(xe @ wg.T) * (xe @ wu.T)) @ wd.T
        np.add.at(y, toks, w64.reshape(-1)[pairs][:, None] * f)
    return dict(ids=ids, weights64=w64, gap=gap, y=y)


def quantization_residual(w_bf16: np.ndarray, signs=None, b: int = 0) -> np.ndarray:
    """Q - W in W's own coordinates, float64: Q the NVFP4 RTN of W (b = 0), or of bf16(W R)
    mapped back by R^T (R = D blockdiag(H_b) / sqrt(b) is orthogonal, so R^T undoes it)."""
    w = bf16_to_f32(w_bf16).astype(np.float64)
    if not b:
        return nvfp4.dequantize_packed(*nvfp4.quantize_weight(w.astype(np.float32))) - w
    wr = bf16_to_f32(rotate_bf16(w_bf16, signs, b))
    q = nvfp4.dequantize_packed(*nvfp4.quantize_weight(wr))
    n = w.shape[-1]
    hb = sylvester(b) / np.sqrt(b)  # symmetric: its transpose is itself
    back = (q.reshape(*q.shape[:-1], n // b, b) @ hb.T).reshape(q.shape) * np.asarray(signs, np.float64)
    return back - w
