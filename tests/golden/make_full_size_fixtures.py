"""Write the oracle's full-size reference values under tests/golden/ (calls only oracle/).

For each batch workload -- the Zipf-skewed prefill (80 experts, 8192 tokens), the
128-expert outlier layer (8192 tokens) and the long batch (80 experts, 32768
tokens) -- the whole layer runs through ``oracle.moe.moe_layer`` on the seeded
inputs of ``workloads.gen``, and two things are stored:

* ``<workload>_y_sketch.npz``: for every token t, ||y_t||_2 and y_t . r_i for the
  four seeded directions r_i of ``workloads.gen.projection_vectors`` (float64),
  plus the per-expert pair counts.  A GPU output that differs from the oracle's
  on any token moves its projections;
* for the long batch, ``long_reap_saliency.json``: the REAP saliency of every
  expert, the mean over its routed tokens of topk_weight * ||f_e(x)||_2 with the
  renormalized sigmoid-and-bias routing weights including routed_scaling_factor
  ('K-EXAONE-152B-A23B-REAP-80E-BF16' model card, 'Pruning Setup').

Run from the repository root (about a quarter of an hour on 8 cores):
    python tests/golden/make_full_size_fixtures.py [workload ...]
"""

from __future__ import annotations

import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import moe as omoe  # noqa: E402
from workloads import by_name, gen  # noqa: E402

OUT_DIR = os.path.dirname(os.path.abspath(__file__))
WORKLOADS = ("prefill_zipf", "outlier_128e", "long_reap")


def run(name: str, threads: int) -> None:
    cfg = by_name(name)
    ws = cfg.weights
    t0 = time.time()
    x = gen.tokens(cfg)
    wr, bias = gen.router_weight(ws), gen.router_bias(cfg)
    gs_x, gs_h = gen.global_scales(ws)

    def ptq(item):
        e, g, u, d = item
        f32 = gen.bf16_bits_to_f32
        return e, omoe.quantize_expert(f32(g), f32(u), f32(d))

    experts = {}
    with ThreadPoolExecutor(threads) as ex:
        for e, q in ex.map(ptq, gen.iter_experts_bf16(ws, threads=2)):
            experts[e] = q
    print(f"{name}: oracle RTN of {len(experts)} experts in {time.time() - t0:.0f} s", flush=True)
    out = omoe.moe_layer(x, wr, bias, cfg.k, cfg.rsf, gs_x, lambda e: experts[e], gs_h, threads=threads)
    y = out["y"]
    counts = np.bincount(out["ids"].reshape(-1), minlength=cfg.E)
    r = gen.projection_vectors(cfg.H)
    np.savez(os.path.join(OUT_DIR, f"{name}_y_sketch.npz"), norm=np.linalg.norm(y, axis=1), proj=y @ r,
             counts=counts.astype(np.int64), T=cfg.T, H=cfg.H, E=cfg.E, k=cfg.k)
    print(f"{name}: layer in {time.time() - t0:.0f} s; wrote {name}_y_sketch.npz", flush=True)
    if cfg.reap:
        payload = {
            "what": "oracle REAP saliency of the long-batch workload (E80 top-8 H6144 I2048 T32768), all routed pairs",
            "source": "'K-EXAONE-152B-A23B-REAP-80E-BF16' model card, 'Pruning Setup': mean(topk_weight * ||f_e(x)||_2)",
            "written_by": "python tests/golden/make_full_size_fixtures.py (calls oracle/ only)",
            "E": cfg.E,
            "T": cfg.T,
            "k": cfg.k,
            "counts": [int(c) for c in counts],
            "saliency_f64_hex": [float(v).hex() for v in out["saliency"]],
        }
        with open(os.path.join(OUT_DIR, "long_reap_saliency.json"), "w") as f:
            json.dump(payload, f, indent=1)
            f.write("\n")
        print(f"{name}: wrote long_reap_saliency.json", flush=True)


def main(argv) -> int:
    names = argv or list(WORKLOADS)
    threads = min(8, len(os.sched_getaffinity(0)))
    for n in names:
        if n not in WORKLOADS:
            raise SystemExit(f"unknown workload {n}; choose from {WORKLOADS}")
        run(n, threads)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
