"""Shared expert and the MoE block output (oracle).

What the pages fix:

* "K-EXAONE-152B-A23B-REAP-80E-NVFP4" model card, section "Quantization
  Setup": the shared experts are among the modules kept in BF16 -- only the
  routed experts are NVFP4;
* "K-EXAONE-152B-A23B-REAP-80E-BF16" model card, section "Pruning Setup":
  pruning removes routed experts only; the shared expert is kept whole.

Readings (pages silent):

* one shared expert per MoE block, a SwiGLU MLP like a routed expert:
  s(x) = h W_down^T with h = silu(x W_gate^T) * (x W_up^T), every token
  passing through it (no routing weight);
* its intermediate size is a parameter (the workloads use the routed
  expert's, 2048);
* x and the weights are BF16; the matmuls are exact float64 here; h is
  rounded once, to BF16 round-to-nearest-even, because it is the input of
  the BF16 down Linear;
* the block output is y_t = (routed combine)_t + s(x_t).

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

from __future__ import annotations

import numpy as np

from .moe import bf16_to_f32, silu


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest BF16 value (ties to even), returned as float64.

    BF16 keeps 8 significant bits and float32's exponent range; below the
    smallest normal (2^-126) the grid step is 2^-133."""
    a = np.asarray(a, dtype=np.float64)
    out = np.zeros_like(a)
    fin = np.isfinite(a) & (a != 0.0)
    _, e = np.frexp(a[fin])  # |a| in [2^(e-1), 2^e)
    step_exp = np.maximum(e - 1, -126) - 7  # exponent of the spacing of the 8-bit significand
    out[fin] = np.ldexp(np.rint(np.ldexp(a[fin], -step_exp)), step_exp)  # np.rint: ties to even
    out[~fin] = a[~fin]
    big = np.abs(out) > 3.3895313892515355e38  # past the largest finite BF16: round to infinity
    out[big] = np.copysign(np.inf, out[big])
    return out


def shared_hidden(x_bf16: np.ndarray, wg_bf16: np.ndarray, wu_bf16: np.ndarray) -> np.ndarray:
    """h = bf16(silu(x W_gate^T) * (x W_up^T)) as float64 [T, I_s]; matmuls in float64."""
    x = bf16_to_f32(x_bf16).astype(np.float64)
    g = x @ bf16_to_f32(wg_bf16).astype(np.float64).T
    u = x @ bf16_to_f32(wu_bf16).astype(np.float64).T
    return round_bf16(silu(g) * u)


def shared_expert(x_bf16: np.ndarray, wg_bf16: np.ndarray, wu_bf16: np.ndarray,
                  wd_bf16: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """(s(x) float64 [T, H], h float64 [T, I_s]) for BF16 bit patterns x [T, H],
    W_gate / W_up [I_s, H] and W_down [H, I_s]."""
    h = shared_hidden(x_bf16, wg_bf16, wu_bf16)
    return h @ bf16_to_f32(wd_bf16).astype(np.float64).T, h


def block_output(y_routed: np.ndarray, shared_out: np.ndarray) -> np.ndarray:
    """The MoE block output: routed combine plus the shared expert, float64."""
    return np.asarray(y_routed, np.float64) + np.asarray(shared_out, np.float64)
