"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

For each of the decode (80 experts, 16 tokens), Zipf-skewed prefill (8192
tokens), 128-expert outlier (8192 tokens) and long-batch REAP (32768 tokens)
workloads:

* routing ids, weights, counts, offsets and the permutation: all tokens,
  bitwise (near-ties, if any, checked for validity);
* activation codes and scales: bitwise on sampled rows;
* weight codes, scales and global scales: bitwise on sampled experts;
* layer output y: rel-L2 <= 2e-3 on sampled tokens (all k experts each);
* one whole expert (every pair routed to it) recomputed by the oracle:
  pair outputs rel-L2 <= 2e-3, per-pair ||f|| and that expert's REAP
  saliency within 1e-3 relative.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from gpu_cases import bf16_round, check_routing, rel_l2, say, to_np, untile_weight_scales
from oracle import moe as omoe
from oracle import nvfp4 as onv
from oracle import reap as oreap
from oracle import routing as oroute
from workloads import CONFIGS, gen

pytestmark = pytest.mark.gpu

THREADS = min(16, len(os.sched_getaffinity(0)))


def _ptq(ws, experts):
    out = {}

    def one(item):
        e, g, u, d = item
        f32 = gen.bf16_bits_to_f32
        return e, omoe.quantize_expert(f32(g), f32(u), f32(d))

    with ThreadPoolExecutor(THREADS) as ex:
        for e, q in ex.map(one, gen.iter_experts_bf16(ws, sorted(experts))):
            out[e] = q
    return out


@pytest.mark.parametrize("ci", [1, 2, 3, 4])
def test_full_size_workload(ci):
    from nvfp4_w4a4_mixture_amd import workload_io

    cfg = CONFIGS[ci]
    ws = cfg.weights
    say(f"full-size workload {ci} {cfg.name}: {cfg.describe()}")
    layer, _ = workload_io.build_layer(cfg)
    xb = gen.tokens(cfg)
    x = workload_io.bf16_to_device(xb, "cuda")
    out = layer(x, out_dtype=torch.float32, reap=True)
    torch.cuda.synchronize()
    say("  GPU layer done")

    # routing, all tokens
    wr, bias = gen.router_weight(ws), gen.router_bias(cfg)
    ids_ref, w32_ref, w64_ref, gap = oroute.route(xb, wr, bias, cfg.k, cfg.rsf)
    ids, w = to_np(out.route.topk_ids), to_np(out.route.topk_w)
    ref = {"ids": ids_ref, "weights64": w64_ref, "gap": gap}
    near = check_routing(ids, w, ref, cfg.rsf, cfg.E)
    print(f"  routing: near-tie tokens {near}, min margin {gap.min():.3e}", flush=True)
    counts, offsets, perm = oroute.permute(ids, cfg.E)
    assert np.array_equal(to_np(out.route.expert_counts), counts)
    assert np.array_equal(to_np(out.route.expert_offsets), offsets)
    assert np.array_equal(to_np(out.route.sorted_pair_ids), perm)
    print(f"  counts: touched {np.count_nonzero(counts)}, min {counts.min()}, max {counts.max()}", flush=True)

    # activation codes on sampled rows
    gs_x, gs_h = gen.global_scales(ws)
    rng = np.random.default_rng(ci)
    rows = np.unique(np.concatenate([[0, cfg.T - 1], rng.integers(0, cfg.T, min(cfg.T, 512))]))
    c_ref, s_ref = onv.quantize(gen.bf16_bits_to_f32(xb[rows]), gs_x)
    rows_d = torch.from_numpy(rows).cuda()
    assert np.array_equal(to_np(out.x_codes[rows_d]), onv.pack_codes(c_ref))
    assert np.array_equal(to_np(out.x_scales[rows_d]), s_ref)

    # experts needed: sampled weight checks, sampled tokens, and one whole expert
    tok = [int(t) for t in rng.choice(cfg.T, 2, replace=False)]
    # the routed expert with the median pair count (bounded oracle work, typical tile raggedness)
    routed = np.nonzero(counts)[0]
    whole = int(routed[np.argsort(counts[routed], kind="stable")[len(routed) // 2]])
    wcheck = {0, cfg.E - 1}
    need = set(wcheck) | set(int(e) for e in ids[tok].reshape(-1)) | {whole}
    experts = _ptq(ws, need)
    say(f"  oracle PTQ of {len(need)} experts done")

    for e in sorted(wcheck):
        q = experts[e]
        c13, s13, g13 = (to_np(t[e]) for t in layer.w13)
        s13 = untile_weight_scales(s13)
        assert np.array_equal(c13[:cfg.I], q.gate_codes) and np.array_equal(c13[cfg.I:], q.up_codes)
        assert np.array_equal(s13[:cfg.I], q.gate_scales) and np.array_equal(s13[cfg.I:], q.up_scales)
        assert g13[0] == q.gate_gs and g13[1] == q.up_gs
        c2, s2, g2 = (to_np(t[e]) for t in layer.w2)
        s2 = untile_weight_scales(s2)
        assert np.array_equal(c2, q.down_codes) and np.array_equal(s2, q.down_scales)
        assert g2 == q.down_gs

    # y on sampled tokens
    ref_tok = omoe.moe_layer(xb, wr, bias, cfg.k, cfg.rsf, gs_x, lambda e: experts[e], gs_h, tokens=tok)
    tok_d = torch.tensor(tok, device="cuda")
    y = to_np(out.y[tok_d])
    err = rel_l2(y, ref_tok["y"])
    print(f"  y rel-L2 on tokens {tok}: {err:.3e}", flush=True)
    assert err <= 2e-3

    # one whole expert: every pair routed to it
    pairs = perm[offsets[whole]:offsets[whole + 1]]
    toks = pairs // cfg.k
    say(f"  whole expert {whole}: {len(pairs)} pairs")
    f = omoe.expert_pairs_output(xb[toks], gs_x, experts[whole], gs_h[whole])
    wp = w64_ref.reshape(-1)[pairs]
    pairs_d = torch.from_numpy(pairs.astype(np.int64)).cuda()
    po = to_np(out.pair_out[pairs_d])
    perr = rel_l2(po, wp[:, None] * f)
    norms = np.linalg.norm(f, axis=1)
    sq = to_np(out.pair_sqnorm[pairs_d]).astype(np.float64)
    nerr = float(np.max(np.abs(np.sqrt(sq) - norms) / norms))
    s_ref = float(np.sum(wp * norms) / len(pairs))
    s_gpu = float(to_np(out.saliency)[whole])
    print(f"  pair_out rel-L2 {perr:.3e}, max ||f|| rel err {nerr:.3e}, saliency {s_gpu:.6g} vs {s_ref:.6g}",
          flush=True)
    assert perr <= 2e-3
    assert nerr <= 1e-3
    assert abs(s_gpu - s_ref) / s_ref <= 1e-3
    # bf16 output of the same step against bf16(oracle)
    out16 = layer(x, out_dtype=torch.bfloat16, reap=False)
    torch.cuda.synchronize()
    err16 = rel_l2(out16.y[tok_d].float().cpu().numpy(), bf16_round(ref_tok["y"]))
    assert err16 <= 2e-3
    if ci == 3:
        _pruned_outlier_layer(cfg, layer, xb, x, wr, bias, gs_x, gs_h)


def _pruned_outlier_layer(cfg, layer, xb, x, wr, bias, gs_x, gs_h):
    """The 128-expert layer pruned to 80 (the REAP one-shot step) with a seeded
    saliency vector given to both sides: kept ids bitwise, the pruned layer's
    routing on all tokens bitwise, y on sampled tokens rel-L2 <= 2e-3."""
    n_keep = 80
    sal = np.random.default_rng(128).random(cfg.E).astype(np.float32)
    say(f"  pruned layer {cfg.E} -> {n_keep} experts")
    pl = layer.prune(torch.from_numpy(sal).cuda(), n_keep)
    out = pl(x, out_dtype=torch.float32)
    torch.cuda.synchronize()
    keep = oreap.keep_ids(sal, n_keep)
    assert np.array_equal(to_np(pl.keep_ids), keep)
    wr_k, b_k = oreap.slice_router(wr, bias, keep)
    ids_ref, _, w64_ref, gap = oroute.route(xb, wr_k, b_k, cfg.k, cfg.rsf)
    ids = to_np(out.route.topk_ids)
    near = check_routing(ids, to_np(out.route.topk_w), {"ids": ids_ref, "weights64": w64_ref, "gap": gap}, cfg.rsf,
                         n_keep)
    counts, offsets, perm = oroute.permute(ids, n_keep)
    assert np.array_equal(to_np(out.route.sorted_pair_ids), perm)
    rng = np.random.default_rng(3)
    tok = [int(t) for t in rng.choice(cfg.T, 2, replace=False)]
    need = set(int(keep[e]) for e in ids[tok].reshape(-1))
    experts = _ptq(cfg.weights, need)
    ref = omoe.moe_layer(xb, wr_k, b_k, cfg.k, cfg.rsf, gs_x, lambda e: experts[int(keep[e])], gs_h[keep],
                         tokens=tok)
    err = rel_l2(to_np(out.y[torch.tensor(tok, device="cuda")]), ref["y"])
    print(f"  pruned: near-tie tokens {near}, touched {np.count_nonzero(counts)}, y rel-L2 on {tok}: {err:.3e}",
          flush=True)
    assert err <= 2e-3
