"""Sigmoid + bias top-k routing, renormalized and scaled, and the expert permutation (oracle).

What the pages fix:

* "K-EXAONE-152B-A23B-REAP-80E-NVFP4" model card, section "Quantization
  Setup" (modules preserved in BF16): the router (``mlp.gate``) is not
  quantized; it acts on the unquantized BF16 hidden state.
* "K-EXAONE-152B-A23B-REAP-80E-BF16" model card, section "Pruning Setup":
  the router has a ``gate.weight`` and an ``e_score_correction_bias``; the
  routing is renormalized sigmoid routing driven by the sigmoid-and-bias
  scores, and ``routed_scaling_factor`` multiplies the routing weights.
* Forum post "1x Spark GB10: 236B unpruned K-EXAONE-236B-A23B ...", sections
  "Caveats" and "Repos": top-8 selection, sigmoid routing.

Readings (pages silent):

* logits are accumulated in float64 (every BF16 x BF16 product is exact in
  float64), so that the top-k decision is taken in one precision on both sides;
* the bias enters the *selection* only: score = sigmoid(logit) + bias picks the
  experts, and the weights renormalize the bias-free sigmoid values,
  w_j = rsf * s_j / sum_{i in selected} s_i (the usual meaning of a
  "correction bias"); no group-limited selection, no epsilon;
* ties in score go to the lower expert index; the k slots are ordered by score,
  descending;
* the permutation is a stable counting sort of pair ids p = t*k + j by expert.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of BF16 bit patterns (uint16)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def router_logits(x_bf16: np.ndarray, w_router_bf16: np.ndarray, chunk: int = 4096) -> np.ndarray:
    """logit[t, e] = sum_h x[t, h] * W_r[e, h], float64 (library matmul as the step)."""
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    w = bf16_bits_to_f64(w_router_bf16)
    T = x_bf16.shape[0]
    out = np.empty((T, w.shape[0]), dtype=np.float64)
    for t0 in range(0, T, chunk):
        out[t0:t0 + chunk] = bf16_bits_to_f64(x_bf16[t0:t0 + chunk]) @ w.T
    return out


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


def select_topk(logits: np.ndarray, bias: np.ndarray, k: int, rsf: float):
    """Top-k selection and renormalized weights from float64 logits.

    Returns ``(ids [T,k] int32, weights [T,k] float32, weights64 [T,k] float64,
    gap [T] float64)`` where ``gap`` is score_(k) - score_(k+1) (inf when k == E),
    the margin by which the k-th choice beat the first excluded expert.
    """
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    s = sigmoid(logits)
    score = s + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    # descending score; a stable sort keeps the lower expert index first on ties
    order = np.argsort(-score, axis=1, kind="stable")
    ids = order[:, :k]
    s_sel = np.take_along_axis(s, ids, axis=1)
    w64 = np.float64(rsf) * s_sel / np.sum(s_sel, axis=1, keepdims=True)
    sorted_scores = np.take_along_axis(score, order, axis=1)
    if k < E:
        gap = sorted_scores[:, k - 1] - sorted_scores[:, k]
    else:
        gap = np.full(T, np.inf)
    return ids.astype(np.int32), w64.astype(np.float32), w64, gap


def route(x_bf16, w_router_bf16, bias, k, rsf):
    """Full routing: float64 logits, then :func:`select_topk`."""
    return select_topk(router_logits(x_bf16, w_router_bf16), bias, k, rsf)


def permute(ids: np.ndarray, E: int):
    """Stable counting sort of pair ids by expert.

    Returns ``(counts [E] int32, offsets [E+1] int32, sorted_pair_ids [T*k] int32)``
    with offsets the exclusive prefix sum of counts and, inside one expert,
    pair ids in increasing order.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_ids = np.argsort(flat, kind="stable")
    return counts, offsets.astype(np.int32), sorted_ids.astype(np.int32)
