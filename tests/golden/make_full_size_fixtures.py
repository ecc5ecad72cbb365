"""Write tests/golden/long_reap_saliency.json: the oracle's REAP saliency vector of
the long-batch workload (80 experts, top-8, hidden 6144, intermediate 2048, 32768
tokens), over all 262,144 routed pairs.

The REAP saliency of expert e is the mean over the tokens routed to e of
topk_weight * ||f_e(x)||_2, with the renormalized sigmoid-and-bias routing
weights including routed_scaling_factor ("K-EXAONE-152B-A23B-REAP-80E-BF16"
model card, "Pruning Setup").  Every value here comes from ``oracle/`` on the
seeded inputs of ``workloads.gen``: FP64 routing, the stable permutation, each
expert's unweighted f through ``oracle.moe.expert_pairs_output`` (the same
arithmetic as ``oracle.moe.moe_layer``), and ``oracle.moe.reap_saliency``.

Run from the repository root (several minutes of CPU):
    python tests/golden/make_long_reap_saliency.py
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
from oracle import routing as oroute  # noqa: E402
from workloads import by_name, gen  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "long_reap_saliency.json")


def main() -> int:
    cfg = by_name("long_reap")
    ws = cfg.weights
    t0 = time.time()
    x = gen.tokens(cfg)
    wr, bias = gen.router_weight(ws), gen.router_bias(cfg)
    gs_x, gs_h = gen.global_scales(ws)
    ids, _, w64, _ = oroute.route(x, wr, bias, cfg.k, cfg.rsf)
    counts, offsets, perm = oroute.permute(ids, cfg.E)
    print(f"routing done in {time.time() - t0:.1f} s; counts {counts.min()}..{counts.max()}", flush=True)
    pair_norm = np.zeros(cfg.T * cfg.k, dtype=np.float64)

    def one(item):
        e, g, u, d = item
        f32 = gen.bf16_bits_to_f32
        q = omoe.quantize_expert(f32(g), f32(u), f32(d))
        pairs = perm[offsets[e]:offsets[e + 1]]
        f = omoe.expert_pairs_output(x[pairs // cfg.k], gs_x, q, gs_h[e])
        return e, pairs, np.sqrt(np.sum(f * f, axis=1))

    threads = min(8, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(threads) as ex:
        for n, (e, pairs, norms) in enumerate(ex.map(one, gen.iter_experts_bf16(ws, threads=2))):
            pair_norm[pairs] = norms
            print(f"  expert {e}: {len(pairs)} pairs ({n + 1}/{cfg.E}, {time.time() - t0:.0f} s)", flush=True)
    sal = omoe.reap_saliency(pair_norm, w64, ids, cfg.E)
    payload = {
        "what": "oracle REAP saliency of the long-batch workload (E80 top-8 H6144 I2048 T32768), all routed pairs",
        "source": "'K-EXAONE-152B-A23B-REAP-80E-BF16' model card, 'Pruning Setup': mean(topk_weight * ||f_e(x)||_2)",
        "written_by": "python tests/golden/make_long_reap_saliency.py (calls oracle/ only)",
        "E": cfg.E,
        "T": cfg.T,
        "k": cfg.k,
        "counts": [int(c) for c in counts],
        "saliency_f64_hex": [float(v).hex() for v in sal],
    }
    with open(OUT, "w") as f:
        json.dump(payload, f, indent=1)
        f.write("\n")
    print(f"wrote {OUT} in {time.time() - t0:.0f} s", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
