"""Write the stored static inputs under ``workloads/static/`` (offline; calls only the oracle).

Two kinds of layer input are not plain random draws:

* the calibrated activation global scales (gs_x, and gs_h[e] for the input of
  each expert's down projection) -- the "K-EXAONE-152B-A23B-REAP-80E-NVFP4"
  model card, section "Quantization Setup", states that activations are
  quantized against calibrated global scales observed during calibration;
* the router bias of the Zipf-skewed prefill workload, fitted so that the
  per-expert pair counts follow a water-filled Zipf(1.1) target.

Both are computed here with the oracle's own arithmetic on the seeded inputs
of ``workloads.gen`` and stored as float32 bit patterns, so that every run on
either side reads identical values.  Run: ``python -m oracle.make_static_inputs
[set ...]`` with set names from ``workloads.configs.WEIGHT_SETS``, ``zipf`` or
``rotation`` (gs_x of the Hadamard-rotated calibration batch of the outlier set).
"""

from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

from workloads import CONFIGS, WEIGHT_SETS, gen

from . import moe, nvfp4, rotation, routing


def _bits(a) -> list[str]:
    return [f"{int(v):08x}" for v in np.asarray(a, dtype=np.float32).reshape(-1).view(np.uint32)]


def _write(name: str, payload: dict) -> None:
    os.makedirs(gen.STATIC_DIR, exist_ok=True)
    path = os.path.join(gen.STATIC_DIR, name)
    with open(path, "w") as f:
        json.dump(payload, f, indent=1)
        f.write("\n")
    print("wrote", path)


def calibration(ws_name: str, threads: int) -> None:
    ws = WEIGHT_SETS[ws_name]
    t0 = time.time()

    def expert(e):
        g, u, d = gen.expert_bf16(ws, e)
        return moe.quantize_expert(gen.bf16_bits_to_f32(g), gen.bf16_bits_to_f32(u), gen.bf16_bits_to_f32(d))

    gs_x, gs_h = moe.calibrate(gen.x_cal(ws), expert, ws.E, threads=threads)
    _write(f"calibration_{ws.name}.json", {
        "what": "static activation global scales 2688/amax over a dense calibration batch",
        "weight_set": ws.name, "n_cal": ws.n_cal,
        "gs_x": float(gs_x), "gs_x_bits": _bits([gs_x])[0],
        "gs_h": [float(v) for v in gs_h], "gs_h_bits": _bits(gs_h),
        "seconds": round(time.time() - t0, 1),
    })


ROTATION_BLOCKS = (16, 128, 2048)


def rotation_calibration(ws_name: str) -> None:
    """gs_x of the Hadamard-rotated calibration batch, one per rotation block size."""
    ws = WEIGHT_SETS[ws_name]
    xc = gen.x_cal(ws)
    s = gen.rotation_signs(ws.H)
    out = {}
    for b in ROTATION_BLOCKS:
        xr = gen.bf16_bits_to_f32(rotation.rotate_bf16(xc, s, b))
        out[str(b)] = _bits([nvfp4.global_scale(np.max(np.abs(xr)))])[0]
    _write(f"rotation_{ws.name}.json", {
        "what": "static gs_x = 2688/amax of the rotated calibration batch, per rotation block size",
        "weight_set": ws.name, "n_cal": ws.n_cal, "gs_x_bits": out,
        "gs_x": {b: float(gen._f32([v])[0]) for b, v in out.items()},
    })


def zipf_bias(cfg_index: int = 2, steps: int = 400) -> None:
    cfg = CONFIGS[cfg_index]
    assert cfg.bias == "zipf"
    ws = cfg.weights
    x = gen.tokens(cfg)
    logits = routing.router_logits(x, gen.router_weight(ws))
    target = gen.zipf_targets(cfg)
    b = gen.router_bias_uniform(ws).astype(np.float64)
    best = None
    for it in range(steps):
        ids, _, _, _ = routing.select_topk(logits, b.astype(np.float32), cfg.k, cfg.rsf)
        n = np.bincount(ids.reshape(-1), minlength=cfg.E).astype(np.float64)
        err = float(np.sum(np.abs(n - target)) / np.sum(target))
        if best is None or err < best[0]:
            best = (err, b.astype(np.float32).copy(), n.copy())
        step = 0.05 if it < steps // 2 else 0.02
        b = np.clip(b + step * (np.log(target) - np.log(np.maximum(n, 0.5))), -2.0, 2.0)
    err, bias, counts = best
    _write(f"zipf_bias_cfg{cfg.index}.json", {
        "what": "router bias fitted so per-expert pair counts follow a water-filled Zipf(1.1) target",
        "config": cfg.index, "fit_l1_rel_error": err,
        "target_counts": [round(float(v), 1) for v in target],
        "realized_counts": [int(v) for v in counts],
        "bias": [float(v) for v in bias], "bias_bits": _bits(bias),
    })


def main(argv) -> None:
    threads = min(8, len(os.sched_getaffinity(0)))
    todo = argv or ["tiny8", "e80", "e128_outlier", "zipf", "rotation"]
    for name in todo:
        if name == "zipf":
            zipf_bias()
        elif name == "rotation":
            rotation_calibration("e128_outlier")
        else:
            calibration(name, threads)


if __name__ == "__main__":
    main(sys.argv[1:])
