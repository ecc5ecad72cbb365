"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This module draws random numbers, rounds them to BF16 and loads the stored
static inputs under ``workloads/static/``.  It holds none of the layer's
arithmetic (no quantization, routing, matmul or activation): both sides take
their inputs from here and compute everything else themselves.

Recipe (per weight set, ``np.random.SeedSequence([0x4E5646, key, stream...])``):

* expert e: float32 N(0, 0.02) draws for W_gate [I, H], W_up [I, H] and
  W_down [H, I] in that order; for the outlier set, each entry is replaced with
  probability 0.005 by a Laplace(0, 0.15) draw; then BF16 round-to-nearest-even;
* router: W_r [E, H] float32 N(0, 0.02) -> BF16; bias float32 U(-0.1, 0.1);
* shared expert: float32 N(0, 0.02) draws for W_gate [I, H], W_up [I, H] and
  W_down [H, I] (intermediate size I of the routed experts, never outliers:
  it stays BF16), then BF16 round-to-nearest-even;
* rotation signs (the diagonal of the Hadamard rotation studied on the outlier
  layer): +-1 with equal probability, one draw per hidden size;
* projection vectors (test data for the full-size output checks): N(0, 1)
  float64 [H, n];
* calibration batch: n_cal tokens of N(0, 1) -> BF16;
* tokens of workload i: N(0, 1) -> BF16, drawn in chunks of 1024 rows, each
  chunk from its own stream so chunks can be drawn in parallel;
* the Zipf-skewed workload replaces the router bias by a stored, fitted bias.
"""

from __future__ import annotations

import json
import os
from concurrent.futures import ThreadPoolExecutor
from functools import lru_cache

import numpy as np

from .configs import LayerConfig, WeightSet

ROOT_KEY = 0x4E5646
STATIC_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "static")
X_CHUNK = 1024

# stream ids inside a weight set
_S_ROUTER_W, _S_ROUTER_B, _S_XCAL, _S_SHARED, _S_EXPERT = 1, 2, 3, 4, 1000
_ROTATION_KEY = 0x524F54
_PROJECTION_KEY = 0x50524A


def _rng(*keys: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([ROOT_KEY, *keys]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """BF16 round-to-nearest-even of float32 values, as uint16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _weight(rng: np.random.Generator, shape, outliers: bool) -> np.ndarray:
    w = rng.standard_normal(shape, dtype=np.float32)
    w *= np.float32(0.02)
    if outliers:
        mask = rng.random(shape, dtype=np.float32) < np.float32(0.005)
        w[mask] = rng.laplace(0.0, 0.15, int(mask.sum())).astype(np.float32)
    return f32_to_bf16_bits(w)


def expert_bf16(ws: WeightSet, e: int):
    """(W_gate [I,H], W_up [I,H], W_down [H,I]) BF16 bit patterns of expert e."""
    rng = _rng(ws.seed_key, _S_EXPERT + e)
    g = _weight(rng, (ws.I, ws.H), ws.outliers)
    u = _weight(rng, (ws.I, ws.H), ws.outliers)
    d = _weight(rng, (ws.H, ws.I), ws.outliers)
    return g, u, d


def shared_expert_bf16(ws: WeightSet):
    """(W_gate [I,H], W_up [I,H], W_down [H,I]) BF16 bit patterns of the shared expert."""
    rng = _rng(ws.seed_key, _S_SHARED)
    return tuple(_weight(rng, shape, False) for shape in ((ws.I, ws.H), (ws.I, ws.H), (ws.H, ws.I)))


def projection_vectors(H: int, n: int = 4) -> np.ndarray:
    """n seeded N(0, 1) vectors of length H, float64 [H, n]: the directions on which the full-size checks
    compare every token's layer output (test data, not part of the layer)."""
    return _rng(_PROJECTION_KEY, H, n).standard_normal((H, n))


def rotation_signs(n: int) -> np.ndarray:
    """The rotation's diagonal: n float32 signs, +1 or -1 with equal probability (one draw per hidden size)."""
    return np.where(_rng(_ROTATION_KEY, n).random(n) < 0.5, -1.0, 1.0).astype(np.float32)


def iter_experts_bf16(ws: WeightSet, experts=None, threads: int | None = None):
    """Yield (e, gate, up, down) for the given experts, drawing several in parallel."""
    experts = list(range(ws.E)) if experts is None else list(experts)
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(threads) as ex:
        # bounded look-ahead keeps host memory at about `threads` experts
        futs = {}
        for i, e in enumerate(experts):
            futs[i] = ex.submit(expert_bf16, ws, e)
            if i >= threads:
                j = i - threads
                yield (experts[j], *futs.pop(j).result())
        for j in sorted(futs):
            yield (experts[j], *futs.pop(j).result())


def router_weight(ws: WeightSet) -> np.ndarray:
    """W_r [E, H] BF16 bit patterns."""
    w = _rng(ws.seed_key, _S_ROUTER_W).standard_normal((ws.E, ws.H), dtype=np.float32)
    return f32_to_bf16_bits(w * np.float32(0.02))


def router_bias_uniform(ws: WeightSet) -> np.ndarray:
    """e_score_correction_bias [E] float32 ~ U(-0.1, 0.1)."""
    return _rng(ws.seed_key, _S_ROUTER_B).uniform(-0.1, 0.1, ws.E).astype(np.float32)


def x_cal(ws: WeightSet) -> np.ndarray:
    """Calibration batch [n_cal, H] BF16 bit patterns, N(0, 1)."""
    x = _rng(ws.seed_key, _S_XCAL).standard_normal((ws.n_cal, ws.H), dtype=np.float32)
    return f32_to_bf16_bits(x)


def _x_chunk(cfg_index: int, H: int, c: int, rows: int) -> np.ndarray:
    x = _rng(0x100 + cfg_index, c).standard_normal((rows, H), dtype=np.float32)
    return f32_to_bf16_bits(x)


def tokens(cfg: LayerConfig, T: int | None = None, threads: int | None = None) -> np.ndarray:
    """Token activations x [T, H] BF16 bit patterns, N(0, 1)."""
    T = cfg.T if T is None else T
    out = np.empty((T, cfg.H), dtype=np.uint16)
    chunks = [(c, c * X_CHUNK, min(T, (c + 1) * X_CHUNK)) for c in range((T + X_CHUNK - 1) // X_CHUNK)]
    threads = threads or min(16, len(os.sched_getaffinity(0)))

    def fill(ch):
        c, a, b = ch
        out[a:b] = _x_chunk(cfg.index, cfg.H, c, X_CHUNK)[: b - a]

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill, chunks))
    return out


def token_rows(cfg: LayerConfig, rows) -> np.ndarray:
    """Selected rows of :func:`tokens` without drawing the whole batch."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), cfg.H), dtype=np.uint16)
    for c in np.unique(rows // X_CHUNK):
        blk = _x_chunk(cfg.index, cfg.H, int(c), X_CHUNK)
        sel = np.nonzero(rows // X_CHUNK == c)[0]
        out[sel] = blk[rows[sel] - c * X_CHUNK]
    return out


# ----------------------------------------------------------------------------
# stored static inputs (written by oracle/make_static_inputs.py)

def _load_json(name: str) -> dict:
    path = os.path.join(STATIC_DIR, name)
    if not os.path.exists(path):
        raise FileNotFoundError(f"static input {path} missing; run `python -m oracle.make_static_inputs`")
    with open(path) as f:
        return json.load(f)


def _f32(values) -> np.ndarray:
    return np.array([np.uint32(int(v, 16)) for v in values], dtype=np.uint32).view(np.float32)


@lru_cache(maxsize=None)
def global_scales(ws: WeightSet):
    """Calibrated static global scales: (gs_x float32, gs_h [E] float32)."""
    d = _load_json(f"calibration_{ws.name}.json")
    gs_x = _f32([d["gs_x_bits"]])[0]
    gs_h = _f32(d["gs_h_bits"])
    assert gs_h.shape == (ws.E,)
    return np.float32(gs_x), gs_h


@lru_cache(maxsize=None)
def rotated_gs_x(ws: WeightSet, block: int) -> np.float32:
    """Calibrated gs_x of the Hadamard-rotated calibration batch (rotation block size `block`)."""
    d = _load_json(f"rotation_{ws.name}.json")
    return np.float32(_f32([d["gs_x_bits"][str(block)]])[0])


def router_bias(cfg: LayerConfig) -> np.ndarray:
    if cfg.bias == "uniform":
        return router_bias_uniform(cfg.weights)
    if cfg.bias == "zipf":
        d = _load_json(f"zipf_bias_cfg{cfg.index}.json")
        b = _f32(d["bias_bits"])
        assert b.shape == (cfg.E,)
        return b
    raise ValueError(cfg.bias)


def zipf_targets(cfg: LayerConfig, s: float = 1.1) -> np.ndarray:
    """Per-expert target pair counts for the Zipf-skewed workload (float64 [E]).

    Pure Zipf is infeasible with top-k routing (one expert can take at most T
    of the T*k pairs), so the target is water-filled:
    c_e = T * min(1, alpha * r_e^-s) with sum c_e = T*k; the ranks r_e are a
    seeded permutation of 1..E.
    """
    E, T, k = cfg.E, cfg.T, cfg.k
    ranks = _rng(0x200 + cfg.index).permutation(E) + 1
    lo, hi = 0.0, float(E) ** s * 10
    for _ in range(200):
        a = 0.5 * (lo + hi)
        tot = np.sum(np.minimum(1.0, a * ranks.astype(np.float64) ** -s)) * T
        if tot > T * k:
            hi = a
        else:
            lo = a
    a = 0.5 * (lo + hi)
    return T * np.minimum(1.0, a * ranks.astype(np.float64) ** -s)
