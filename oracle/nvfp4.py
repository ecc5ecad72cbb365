"""NVFP4 round-to-nearest quantization and dequantization (oracle).

What the pages fix ("K-EXAONE-152B-A23B-REAP-80E-NVFP4" model card, section
"Quantization Setup"; NetsPresso AQ blog, section "The Standard NVFP4 Serving
Spec"):

* elements are FP4 E2M1, one FP8 E4M3 block scale per group of 16 consecutive
  elements along the input (reduction) dimension, plus one FP32 global scale
  per tensor -- the "double-scale structure";
* quantization is round-to-nearest (RTN);
* activations are quantized dynamically (block scales computed at run time)
  against a *calibrated*, static global scale;
* routed expert weights are quantized per expert Linear module.

Readings taken where the pages are silent (each is also pinned by a test):

* the global scale ``gs`` is a multiplier, ``gs = 448 * 6 / amax`` (the E4M3
  maximum times the E2M1 maximum), so a block's ideal scale is
  ``amax_block / 6 * gs`` and dequantization divides by ``gs``;
* every scale step is one IEEE float32 operation, in this order, with no fused
  multiply-add: ``s = f32(f32(a / 6) * gs)``, ``inv = f32(gs / s_d)``,
  ``v = f32(x * inv)``;
* a block whose E4M3 scale rounds to zero encodes all sixteen codes as 0x0;
* the sign bit of a code is the sign bit of ``v`` (so a negative value that
  rounds to magnitude zero is stored as 0x8, "negative zero");
* codes are packed two per byte, element 2j in bits 3:0 and element 2j+1 in
  bits 7:4.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

from __future__ import annotations

import numpy as np

from . import formats

BLOCK = 16
E2M1_MAX = 6.0
E4M3_MAX = 448.0
GS_NUMERATOR = np.float32(E4M3_MAX * E2M1_MAX)  # 2688


def global_scale(amax) -> np.float32:
    """FP32 global scale ``2688 / amax`` (amax of |tensor|); 1.0 when amax is 0."""
    a = np.float32(amax)
    if a == 0:
        return np.float32(1.0)
    return np.float32(GS_NUMERATOR / a)


def quantize(x: np.ndarray, gs) -> tuple[np.ndarray, np.ndarray]:
    """Quantize ``x`` [rows, cols] (cols % 16 == 0) with global scale ``gs``.

    Returns ``(codes, scales)``: ``codes`` is uint8 [rows, cols], one 4-bit
    E2M1 code per element (unpacked), and ``scales`` is uint8 [rows, cols/16],
    one E4M3 byte per block of 16 consecutive elements of a row.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if x.ndim != 2 or x.shape[1] % BLOCK:
        raise ValueError("quantize expects a 2-D array whose column count is a multiple of 16")
    gs = np.float32(gs)
    rows, cols = x.shape
    xb = x.reshape(rows, cols // BLOCK, BLOCK)

    # step 1: block amax (exact: max of float32 magnitudes)
    amax = np.max(np.abs(xb), axis=2)  # float32
    # step 2: ideal scale in float32: s = f32(f32(amax / 6) * gs)
    s = (amax / np.float32(E2M1_MAX)).astype(np.float32)
    s = (s * gs).astype(np.float32)
    # step 3: E4M3 round-to-nearest-even with saturation
    scale_codes = formats.e4m3_encode_nonneg(s)
    s_d = formats.E4M3_VALUES[scale_codes].astype(np.float32)  # exact in f32
    # step 4: per-element code; zero scale -> all-zero codes
    zero_blk = s_d == 0
    safe = np.where(zero_blk, np.float32(1.0), s_d).astype(np.float32)
    inv = (gs / safe).astype(np.float32)  # f32(gs / s_d)
    v = (xb * inv[:, :, None]).astype(np.float32)  # f32(x * inv)
    codes = formats.e2m1_encode(v)
    codes = np.where(zero_blk[:, :, None], np.uint8(0), codes).astype(np.uint8)
    return codes.reshape(rows, cols), scale_codes.astype(np.uint8)


def dequantize(codes: np.ndarray, scales: np.ndarray, gs) -> np.ndarray:
    """float64 values ``e2m1(code) * e4m3(scale) / gs`` for unpacked codes."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, cols = codes.shape
    vals = formats.E2M1_VALUES[codes].reshape(rows, cols // BLOCK, BLOCK)
    sv = formats.E4M3_VALUES[np.asarray(scales, dtype=np.uint8)]
    out = vals * sv[:, :, None] / np.float64(np.float32(gs))
    return out.reshape(rows, cols)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Pack unpacked 4-bit codes [rows, cols] into bytes [rows, cols/2], low nibble first."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] & 0xF) | ((codes[:, 1::2] & 0xF) << 4)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_codes`."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    out = np.empty((rows, half * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def quantize_weight(w: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.float32]:
    """Offline RTN of one Linear weight [out, in]: its own global scale, then :func:`quantize`.

    Returns ``(packed_codes [out, in/2], scales [out, in/16], gs)``.
    """
    w = np.asarray(w, dtype=np.float32)
    gs = global_scale(np.max(np.abs(w)))
    codes, scales = quantize(w, gs)
    return pack_codes(codes), scales, gs


def dequantize_packed(packed: np.ndarray, scales: np.ndarray, gs) -> np.ndarray:
    """float64 dequantization from packed codes."""
    return dequantize(unpack_codes(packed), scales, gs)
