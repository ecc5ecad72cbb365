#!/usr/bin/env python3
"""Benchmark of the routed-expert NVFP4 W4A4 MoE layer on one MI355X.

One step = one pass of the whole layer over one batch of seeded synthetic
tokens: sigmoid+bias top-k routing and the expert permutation, NVFP4
quantization of the activations, gate_up + SwiGLU + re-quantization, down +
weighted scatter with the per-pair sum of squares, the combine, and the REAP
saliency finalize.  Inputs are resident in HBM before the timed region.

Default workload: the largest single-GPU one, the long batch with fused REAP
saliency (80 experts, top-8, hidden 6144, intermediate 2048, 32768 tokens),
MFMA-bound.  The same line carries, under "workloads", short measurements of
the decode (HBM-bound, hot and with the last-level cache flushed between
steps), Zipf-skewed prefill and 128-expert outlier workloads.  Prints one JSON
line.

  python bench.py [--steps K] [--warmup W] [--config N] [--no-cpu-baseline] [--no-extra-workloads]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "routed-MoE layer tokens/sec (NVFP4 W4A4) + % HBM / % MFMA roofline"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
# Extra workloads: untimed busy time before timing (GPU clocks ramp up under load) and the shortest timed region
EXTRA_BUSY_S = 0.2
EXTRA_TIMED_S = 0.05
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense FP16 MFMA
PROFILES = os.path.join(ROOT, "profiles")
FFN_SOURCE = os.path.join(ROOT, "nvfp4_w4a4_mixture_amd", "csrc", "ffn.hip")


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4,
                    help="workload index (0..4); 4 = long batch with fused REAP saliency, the largest")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens in the oracle's timed sample (default: 16 for the decode batch, 4 otherwise)")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="skip the short measurements of the other full-size workloads")
    ap.add_argument("--extra-steps", type=int, default=20, help="timed steps per extra workload")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="MiB written between decode steps for the cold (cache-flushed) measurement")
    ap.add_argument("--union-sweep", action="store_true",
                    help="decode only: time the layer on the first T tokens for T = 1, 2, 4, 8, 16 and report the "
                         "experts touched, weight bytes streamed and tokens/s (one JSON line)")
    ap.add_argument("--reap-prune", type=int, default=0, metavar="N_KEEP",
                    help="REAP one-shot pruning study on --config (3 = the 128-expert layer): saliency from one "
                         "pass, prune to N_KEEP experts, output drift against the unpruned layer for the REAP, a "
                         "seeded random, the lowest-saliency and the most-routed choice, prune time and step times (one JSON line)")
    ap.add_argument("--shared", action="store_true",
                    help="BF16 shared expert and block output study on --config: the shared expert alone against "
                         "its roofline, and the step time of the routed layer, of the block with the shared expert "
                         "on its own stream, and of the block run serially (one JSON line)")
    ap.add_argument("--rotation", action="store_true",
                    help="offline Hadamard rotation study on --config: time the rotation of every W_gate/W_up row and "
                         "of the tokens for block sizes 16, 128 and 2048 against the HBM roofline (one JSON line)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times) to calibrate HBM counters")
    return ap.parse_args(argv)


def copy_probe(mib: int) -> int:
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": n * 4, "copies": 3}), flush=True)
    return 0


def ffn_source_hash() -> str:
    with open(FFN_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stage_bytes_flops(cfg, counts):
    """Algorithmic bytes and FLOPs of the two FFN stages for one launch."""
    import numpy as np

    H, I, T, k = cfg.H, cfg.I, cfg.T, cfg.k
    touched = int(np.count_nonzero(counts))
    pairs = T * k
    nv = 0.5625  # bytes per NVFP4 element: 4-bit code + one E4M3 byte per 16
    w13 = 2 * I * H * nv
    w2 = H * I * nv
    gate_up_bytes = touched * w13 + T * H * nv + pairs * I * nv  # weights + x codes + h codes out
    # weights + h codes + pair rows (FP16 values and one FP32 scale per row)
    down_bytes = touched * w2 + pairs * I * nv + pairs * (H * 2 + 4)
    return dict(touched=touched,
                gate_up=dict(bytes=gate_up_bytes, flops=2.0 * pairs * H * 2 * I, per_expert_bytes=w13),
                down=dict(bytes=down_bytes, flops=2.0 * pairs * I * H, per_expert_bytes=w2))


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it matches the current kernel source."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    h = re.search(r"ffn_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or not h or h.group(1) != ffn_source_hash():
        return None
    return float(m.group(1))


def union_sweep(cfg, layer, x, steps: int, warmup: int) -> dict:
    """Small-batch decode: the union of the experts the T tokens touch sets the bytes streamed per step."""
    import numpy as np
    import torch

    per_expert = stage_bytes_flops(cfg, np.ones(cfg.E))["gate_up"]["per_expert_bytes"] + \
        stage_bytes_flops(cfg, np.ones(cfg.E))["down"]["per_expert_bytes"]
    rows = []
    for T in (1, 2, 4, 8, 16):
        if T > x.shape[0]:
            break
        xt = x[:T].contiguous()
        for _ in range(warmup):
            layer(xt, out_dtype=torch.bfloat16, reap=False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            out = layer(xt, out_dtype=torch.bfloat16, reap=False)
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / steps
        touched = int(np.count_nonzero(out.route.expert_counts.cpu().numpy()))
        wbytes = touched * per_expert
        rows.append({"tokens": T, "experts_touched": touched, "weight_bytes": int(wbytes), "ms_per_step": sec * 1e3,
                     "tokens_per_s": T / sec, "weight_GB_per_s": wbytes / sec / 1e9})
    return {"study": "decode expert union", "workload": cfg.name, "steps": steps, "warmup": warmup, "rows": rows}


def _step_ms(layer, x, steps: int, warmup: int) -> float:
    import torch

    for _ in range(warmup):
        layer(x, out_dtype=torch.bfloat16, reap=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer(x, out_dtype=torch.bfloat16, reap=False)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


def reap_prune_study(cfg, layer, x, n_keep: int, steps: int, warmup: int) -> dict:
    """REAP one-shot pruning: rank the saliency of one pass, keep n_keep experts, measure the output drift."""
    import numpy as np
    import torch

    from nvfp4_w4a4_mixture_amd import ops

    full = layer(x, out_dtype=torch.float32, reap=True)
    y_full = full.y.clone()
    sal = full.saliency.clone()
    counts = full.route.expert_counts.cpu().numpy()
    torch.cuda.synchronize()
    # time the pruning itself: the selection and the gathers of every per-expert tensor
    prune_ms = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pl = layer.prune(sal, n_keep)
        e1.record()
        torch.cuda.synchronize()
        prune_ms.append(e0.elapsed_time(e1))
    tensors = [pl.w_router, pl.bias, pl.h_gs, *pl.w13, *pl.w2]
    moved = sum(t.numel() * t.element_size() for t in tensors)
    keeps = {"reap": pl.keep_ids}
    rng = np.random.default_rng(n_keep)
    keeps["random"] = torch.from_numpy(np.sort(rng.choice(cfg.E, n_keep, replace=False)).astype(np.int32)).cuda()
    keeps["lowest_saliency"] = torch.from_numpy(
        np.sort(np.argsort(sal.cpu().numpy(), kind="stable")[:n_keep]).astype(np.int32)).cuda()
    # frequency pruning, for contrast: keep the experts that receive the most pairs
    keeps["most_routed"] = torch.from_numpy(
        np.sort(np.argsort(-counts, kind="stable")[:n_keep]).astype(np.int32)).cuda()
    den = torch.linalg.vector_norm(y_full.double())
    rows = []
    for name, keep in keeps.items():
        p = pl if name == "reap" else layer.take_experts(keep)
        out = p(x, out_dtype=torch.float32)
        drift = float(torch.linalg.vector_norm(out.y.double() - y_full.double()) / den)
        kept = np.zeros(cfg.E, bool)
        kept[keep.cpu().numpy()] = True
        rows.append({"choice": name, "y_rel_l2_drift": drift,
                     "pairs_rerouted_frac": float(counts[~kept].sum() / counts.sum()),
                     "kept_saliency_sum_frac": float(sal.cpu().numpy()[kept].sum() / sal.cpu().numpy().sum())})
        del p, out
    ms_full = _step_ms(layer, x, steps, warmup)
    ms_pruned = _step_ms(pl, x, steps, warmup)
    return {"study": "REAP one-shot pruning", "workload": cfg.name, "experts": cfg.E, "kept": n_keep,
            "tokens": cfg.T, "prune_ms": float(np.median(prune_ms)), "prune_bytes_gathered": int(moved),
            "prune_GB_per_s_rw": 2 * moved / (np.median(prune_ms) / 1e3) / 1e9, "rows": rows,
            "step_ms_unpruned": ms_full, "step_ms_pruned": ms_pruned,
            "tokens_per_s_unpruned": cfg.T / ms_full * 1e3, "tokens_per_s_pruned": cfg.T / ms_pruned * 1e3,
            "steps": steps, "warmup": warmup}


def shared_study(cfg, layer, x, steps: int, warmup: int) -> dict:
    """The BF16 shared expert beside the routed path: its own roofline and what it adds to a step."""
    import torch

    from nvfp4_w4a4_mixture_amd import ops, workload_io

    w13, w2 = workload_io.shared_expert(cfg.weights, x.device)
    layer.set_shared_expert(w13, w2)
    T, H, I = x.shape[0], cfg.H, cfg.I
    out = torch.empty((T, H), dtype=torch.float32, device=x.device)
    ws = torch.empty((max(ops.moe_shared_workspace_bytes(T, H, I), 1),), dtype=torch.uint8, device=x.device)
    for _ in range(warmup):
        ops.moe_shared_expert(x, w13, w2, out=out, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        ops.moe_shared_expert(x, w13, w2, out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms_shared = e0.elapsed_time(e1) / steps
    wbytes = 3 * I * H * 2
    flops = 2 * T * H * I * 3
    if cfg.bound == "mfma":
        achieved = flops / (ms_shared / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_F16_PEAK_TFLOPS, "dtype": "bf16"}
    else:
        nbytes = wbytes + T * H * 2 + T * H * 4
        achieved = nbytes / (ms_shared / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}

    def step_ms(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e3

    def serial():
        ops.moe_shared_expert(x, w13, w2, out=out, workspace=ws)
        o = layer(x, out_dtype=torch.bfloat16, reap=False)
        ops.moe_combine_block(o.pair_out, o.pair_scale, out, T, cfg.k, torch.bfloat16, y=o.y)

    ms_routed = step_ms(lambda: layer(x, out_dtype=torch.bfloat16, reap=False))
    ms_block = step_ms(lambda: layer(x, out_dtype=torch.bfloat16, reap=False, block=True))
    ms_serial = step_ms(serial)
    return {"study": "shared expert and block output", "workload": cfg.name, "tokens": T, "hidden": H,
            "shared_intermediate": I, "shared_ms": ms_shared, "shared_weight_bytes": wbytes, "shared_flops": flops,
            "shared_roofline": roof, "step_ms_routed": ms_routed, "step_ms_block_two_streams": ms_block,
            "step_ms_block_serial": ms_serial, "tokens_per_s_block": T / ms_block * 1e3,
            "steps": steps, "warmup": warmup}


def rotation_study(cfg, x, steps: int, warmup: int) -> dict:
    """The offline rotation kernel on the layer's W13 rows and tokens: time and HBM rate per block size."""
    import torch

    from nvfp4_w4a4_mixture_amd import ops, workload_io
    from workloads import gen

    ws = cfg.weights
    w13, _ = workload_io.expert_weights_bf16(ws, x.device)
    w = w13.view(-1, ws.H)
    out = torch.empty_like(w)
    xo = torch.empty_like(x)
    s = torch.from_numpy(gen.rotation_signs(ws.H)).to(x.device)
    rows = []
    for blk in (16, 128, 2048):
        for name, src, dst in (("w13", w, out), ("tokens", x, xo)):
            for _ in range(max(1, warmup)):
                ops.hadamard_rotate_bf16(src, s, blk, out=dst)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = max(1, steps)
            e0.record()
            for _ in range(n):
                ops.hadamard_rotate_bf16(src, s, blk, out=dst)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / n
            nbytes = 2 * src.numel() * 2  # BF16 read and written once
            rows.append({"block": blk, "operand": name, "rows": src.shape[0], "cols": src.shape[1], "ms": ms,
                         "GB_per_s": nbytes / (ms / 1e3) / 1e9, "hbm_frac": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS})
    return {"study": "offline Hadamard rotation kernel", "workload": cfg.name, "rows": rows, "steps": steps,
            "warmup": warmup}


def cpu_baseline(cfg, n_tokens: int) -> dict:
    """The oracle on a bounded sample of the same workload (the first n_tokens tokens)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    from oracle import moe as omoe
    from oracle import routing as oroute
    from workloads import gen

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    ws = cfg.weights
    rows = list(range(n_tokens))
    x = gen.token_rows(cfg, rows)
    wr = gen.router_weight(ws)
    bias = gen.router_bias(cfg)
    gs_x, gs_h = gen.global_scales(ws)
    # offline part (not timed): which experts the sample needs, and their RTN weights
    ids, _, _, _ = oroute.route(x, wr, bias, cfg.k, cfg.rsf)
    need = sorted(set(int(e) for e in ids.reshape(-1)))
    experts = {}

    def ptq(item):
        e, g, u, d = item
        f32 = gen.bf16_bits_to_f32
        return e, omoe.quantize_expert(f32(g), f32(u), f32(d))

    with ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
        for e, q in ex.map(ptq, gen.iter_experts_bf16(ws, need)):
            experts[e] = q
    # the layer on the sample, repeated until about 10 s of CPU work (at most 5 passes)
    reps, dt = 0, 0.0
    while reps < 5 and (reps == 0 or dt < 10.0):
        t0 = time.perf_counter()
        out = omoe.moe_layer(x, wr, bias, cfg.k, cfg.rsf, gs_x, lambda e: experts[e], gs_h)
        dt += time.perf_counter() - t0
        reps += 1
        assert np.isfinite(out["y"]).all()
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except Exception:  # pragma: no cover
        pass
    return {"value": n_tokens * reps / dt, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"first {n_tokens} tokens of the same batch ({len(need)} experts touched), full layer incl. "
                      f"routing, quantization, fp64 expert FFN over dequantized operands, combine and REAP; "
                      f"{reps} pass{'es' if reps > 1 else ''} in {dt:.2f} s; offline RTN of the weights not timed; host CPU: {cpu}"}


def layer_bytes_flops(cfg, counts):
    """Algorithmic bytes and FLOPs of one whole-layer step: every touched expert's NVFP4 weights, the BF16
    router, x in and y out (BF16); the FFN FLOPs (2 H 2I + 2 I H per pair) plus the router's 2 T H E."""
    import numpy as np

    touched = int(np.count_nonzero(counts))
    nv = 0.5625
    wbytes = touched * (3 * cfg.I * cfg.H * nv)
    nbytes = wbytes + cfg.E * cfg.H * 2 + cfg.T * cfg.H * 2 + cfg.T * cfg.H * 2
    flops = 2.0 * cfg.pairs * (cfg.H * 2 * cfg.I + cfg.I * cfg.H) + 2.0 * cfg.T * cfg.H * cfg.E
    return dict(bytes=nbytes, flops=flops, touched=touched)


def _roof(bound: str, work: float, seconds: float) -> dict:
    if bound == "mfma":
        a = work / seconds / 1e12
        return {"bound": "mfma", "achieved": a, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": a / MFMA_F16_PEAK_TFLOPS}
    a = work / seconds / 1e9
    return {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": a / HBM_PEAK_GBS}


def _busy_steps(layer, x, reap: bool, seconds: float) -> tuple:
    """Untimed steps until the GPU has run them for `seconds` of wall time (in chunks, each ended by a
    device synchronization, so the host never queues far ahead).  Returns (steps run, seconds per step)."""
    import torch

    n, t0, chunk = 0, time.perf_counter(), 4
    while True:
        for _ in range(chunk):
            layer(x, out_dtype=torch.bfloat16, reap=reap)
        torch.cuda.synchronize()
        n += chunk
        dt = time.perf_counter() - t0
        if dt >= seconds:
            return n, dt / n
        chunk = min(2 * chunk, 256)


def measure(cfg, layer, x, steps: int, warmup: int, reap: bool, min_busy_s: float = 0.0,
            min_timed_s: float = 0.0) -> dict:
    """Time `steps` whole-layer steps (after `warmup` untimed ones) on the current stream.

    The warm-up steps record HIP events around every stage (stage_ms_warmup) and pick the dominant FFN
    stage.  The timed region is `steps` steps with no events at all (each event recorded on the stream
    adds a gap), bracketed by device synchronizations: that wall time per step is the figure reported.
    A second pass of `steps` steps records events only around the dominant stage, for its kernel time.

    min_busy_s > 0 adds untimed steps after the warm-up until the GPU has been busy for that long: its
    clocks drop while it idles and take milliseconds of load to come back, longer than a few short
    decode steps.  min_timed_s > 0 raises the number of timed steps so that the timed region lasts about
    that long.  Both stay 0 for the headline, which runs exactly `warmup` and `steps` steps.
    Returns the wall time per step, the steps and warm-up steps run, the dominant kernel's mean event
    time and the routing counts of the last step."""
    import numpy as np
    import torch

    stages = layer.STAGES
    wev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(max(warmup, 1))]
    for i in range(max(warmup, 1)):
        layer(x, out_dtype=torch.bfloat16, reap=reap, events=wev[i])
    torch.cuda.synchronize()
    skip = min(2, len(wev) - 1)  # the first steps allocate and load
    ms_stage = {s: float(np.mean([ev[j].elapsed_time(ev[j + 1]) for ev in wev[skip:]])) for j, s in enumerate(stages)}
    dom = "gate_up" if ms_stage["gate_up"] >= ms_stage["down"] else "down"
    j_dom = stages.index(dom)
    warm_run = max(warmup, 1)
    if min_busy_s > 0:
        n_busy, est = _busy_steps(layer, x, reap, min_busy_s)
        warm_run += n_busy
        if min_timed_s > 0:
            steps = max(steps, int(np.ceil(min_timed_s / est)))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        out = layer(x, out_dtype=torch.bfloat16, reap=reap)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    # the dominant kernel's time, from events around its stage only, in a pass of its own
    events = [[None] * (len(stages) + 1) for _ in range(steps)]
    for ev in events:
        ev[j_dom], ev[j_dom + 1] = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(steps):
        out = layer(x, out_dtype=torch.bfloat16, reap=reap, events=events[i])
    torch.cuda.synchronize()
    dom_ms = float(np.mean([ev[j_dom].elapsed_time(ev[j_dom + 1]) for ev in events]))
    counts = out.route.expert_counts.cpu().numpy()
    return dict(sec_per_step=sec, dom=dom, dom_ms=dom_ms, ms_stage=ms_stage, counts=counts, steps=steps,
                warmup=warm_run)


def roofline_of(cfg, m: dict) -> dict:
    """The dominant kernel against its roofline (algorithmic work / its event time), the traffic the
    committed counter summary gives for that kernel and workload, and the whole layer against the same
    roofline on the wall clock of the timed steps."""
    bf = stage_bytes_flops(cfg, m["counts"])
    dom = m["dom"]
    bound = "mfma" if cfg.bound == "mfma" else "hbm"
    work = bf[dom]["flops"] if bound == "mfma" else bf[dom]["bytes"]
    roof = _roof(bound, work, m["dom_ms"] / 1e3)
    kernel = {"gate_up": "ffn_gate_up", "down": "ffn_down"}[dom]
    roof["traffic"] = read_traffic(kernel, cfg.name)
    roof["kernel"] = kernel
    roof["kernel_ms"] = m["dom_ms"]
    roof["algorithmic_bytes"] = bf[dom]["bytes"]
    roof["algorithmic_flops"] = bf[dom]["flops"]
    lb = layer_bytes_flops(cfg, m["counts"])
    lw = lb["flops"] if bound == "mfma" else lb["bytes"]
    layer_roof = _roof(bound, lw, m["sec_per_step"])
    roof["layer"] = {"achieved": layer_roof["achieved"], "frac": layer_roof["frac"],
                     "algorithmic_bytes" if bound == "hbm" else "algorithmic_flops": lw,
                     "ms_per_step": m["sec_per_step"] * 1e3}
    return roof


def decode_cold_hot(cfg, layer, x, steps: int, warmup: int, flush_mib: int, reap: bool) -> dict:
    """The decode layer per step (HIP events around each whole step), hot and with a flush_mib MiB buffer
    read between steps so that no weight bytes stay in the last-level cache (256 MB on MI355X).  The
    flush reads (a sum) rather than writes, so no dirty lines are left to write back during the step."""
    import numpy as np
    import torch

    scratch = torch.ones(flush_mib * (1 << 20) // 4, dtype=torch.float32, device=x.device)
    res = {}
    for mode in ("hot", "cold"):
        for _ in range(warmup):
            layer(x, out_dtype=torch.bfloat16, reap=reap)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            if mode == "cold":
                scratch.sum()
            ev[i][0].record()
            out = layer(x, out_dtype=torch.bfloat16, reap=reap)
            ev[i][1].record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
        lb = layer_bytes_flops(cfg, out.route.expert_counts.cpu().numpy())
        res[mode] = {"us_per_step_median": ms * 1e3, "tokens_per_s": cfg.T / (ms / 1e3),
                     "hbm_frac": lb["bytes"] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS}
    res["flush_bytes"] = flush_mib * (1 << 20)
    res["layer_bytes"] = lb["bytes"]
    del scratch
    return res


def extra_workloads(main_cfg, main_layer, steps: int, warmup: int, flush_mib: int) -> dict:
    """Short measurements of the other full-size workloads, each against its own roofline."""
    import torch

    from nvfp4_w4a4_mixture_amd import workload_io
    from nvfp4_w4a4_mixture_amd.layer import NVFP4MoELayer
    from workloads import CONFIGS, gen

    out = {}
    for cfg in CONFIGS[1:]:
        if cfg.index == main_cfg.index:
            continue
        if cfg.weights == main_cfg.weights:  # the same expert weights: share them, with this workload's bias
            bias = torch.from_numpy(gen.router_bias(cfg)).to(main_layer.device)
            layer = NVFP4MoELayer(main_layer.w_router, bias, cfg.k, cfg.rsf, main_layer.x_gs, main_layer.h_gs,
                                  *main_layer.w13, *main_layer.w2)
        else:
            layer, _ = workload_io.build_layer(cfg, main_layer.device)
        x = workload_io.tokens(cfg, main_layer.device)
        # each extra workload follows seconds of host-side set-up with the GPU idle: warm it up by busy time
        m = measure(cfg, layer, x, steps, warmup, reap=cfg.reap, min_busy_s=EXTRA_BUSY_S, min_timed_s=EXTRA_TIMED_S)
        roof = roofline_of(cfg, m)
        rec = {"workload": f"{cfg.name}: {cfg.describe()}", "reap": cfg.reap, "tokens_per_s": cfg.T / m["sec_per_step"],
               "ms_per_step": m["sec_per_step"] * 1e3, "touched_experts": int((m["counts"] > 0).sum()),
               "stage_ms_warmup": m["ms_stage"], "roofline": roof, "steps": m["steps"], "warmup": m["warmup"]}
        if cfg.name == "decode":
            rec["per_step_events"] = decode_cold_hot(cfg, layer, x, m["steps"], warmup, flush_mib, cfg.reap)
        out[cfg.name] = rec
        del layer, x
        torch.cuda.empty_cache()
    return out


def main(argv=None) -> int:
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this layer runs on exactly one GPU; --gpus must be 1 "
                                   "(expert-parallel sharding over several GPUs is not built)"}), flush=True)
        return 2
    if args.copy_probe:
        return copy_probe(args.copy_probe)
    import torch

    from nvfp4_w4a4_mixture_amd import workload_io
    from workloads import CONFIGS

    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    t_setup = time.perf_counter()
    layer, _ = workload_io.build_layer(cfg, dev)
    x = workload_io.tokens(cfg, dev)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    if args.union_sweep:
        print(json.dumps(union_sweep(cfg, layer, x, args.steps, args.warmup)), flush=True)
        return 0
    if args.rotation:
        del layer
        print(json.dumps(rotation_study(cfg, x, args.steps, args.warmup)), flush=True)
        return 0
    if args.shared:
        print(json.dumps(shared_study(cfg, layer, x, args.steps, args.warmup)), flush=True)
        return 0
    if args.reap_prune:
        print(json.dumps(reap_prune_study(cfg, layer, x, args.reap_prune, args.steps, args.warmup)), flush=True)
        return 0

    # the headline: every step runs the whole layer with the REAP saliency
    m = measure(cfg, layer, x, args.steps, args.warmup, reap=True)
    roof = roofline_of(cfg, m)
    rec = {
        "metric": METRIC,
        "value": cfg.T / m["sec_per_step"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["sec_per_step"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.describe()}, NVFP4 W4A4 (E2M1 x E4M3/16 + fp32 global), "
                               f"routed_scaling_factor {cfg.rsf}, REAP saliency every step",
                   "operands": "nvfp4 codes decoded in registers to f16 for MFMA, f32 accumulate; routing in f64",
                   "tokens_per_step": cfg.T, "experts": cfg.E, "top_k": cfg.k, "hidden": cfg.H,
                   "intermediate": cfg.I, "touched_experts": int((m["counts"] > 0).sum())},
        "stage_ms_warmup": m["ms_stage"],
        "roofline": roof,
        "setup_s": round(setup_s, 1),
    }
    print(f"# headline done: {rec['value']:.0f} tokens/s, {rec['ms_per_step']:.3f} ms/step", file=sys.stderr,
          flush=True)
    if not args.no_extra_workloads:
        rec["workloads"] = extra_workloads(cfg, layer, args.extra_steps, min(args.warmup, 5), args.flush_mib)
        print("# extra workloads done", file=sys.stderr, flush=True)
    del layer, x
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        n = args.cpu_tokens or (16 if cfg.T <= 16 else 4)
        rec["cpu_baseline"] = cpu_baseline(cfg, min(n, cfg.T))
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
