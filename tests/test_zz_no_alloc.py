"""moe_nvfp4_grouped_ffn_noalloc (the grouped FFN on the library's static scratch,
for callers that cannot allocate) against moe_nvfp4_grouped_ffn with a caller
workspace: pair rows (FP16 values and row scales) and sums of squares bitwise equal, on calls in a row
whose inputs shrink (the tiled kernels, then the decode kernels), so the second
and third calls run on scratch the earlier ones left behind."""

import numpy as np
import pytest
import torch

from gpu_cases import dev_bf16, gpu_layer, random_case, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    from nvfp4_w4a4_mixture_amd import ops

    return ops


def test_noalloc_matches_workspace_call_on_shrinking_inputs(ops):
    for name, seed, T in (("noalloc_tiled", 71, 300), ("noalloc_tiled_small", 72, 40), ("noalloc_decode", 73, 12)):
        case = random_case(name, seed, T, 512, 256, 16, 4)
        say(f"{name}: T={T} H={case.H} I={case.I} E={case.E} k={case.k}")
        layer = gpu_layer(case)
        r, xc, xs = ops.moe_route_quantize(dev_bf16(case.x), layer.w_router, layer.bias, case.k, case.rsf, layer.x_gs)
        n, H = T * case.k, case.H
        po_ref = torch.empty((n, H), dtype=torch.float16, device="cuda")
        ps_ref = torch.empty((n,), dtype=torch.float32, device="cuda")
        sq_ref = torch.empty((n,), dtype=torch.float32, device="cuda")
        ops.moe_nvfp4_grouped_ffn(xc, xs, layer.x_gs, *layer.w13, *layer.w2, layer.h_gs, case.k, r.expert_offsets,
                                  r.sorted_pair_ids, r.topk_w, pair_out=po_ref, pair_scale=ps_ref, pair_sqnorm=sq_ref)
        po = torch.full((n, H), float("nan"), dtype=torch.float16, device="cuda")
        ps = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        sq = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        ops.moe_nvfp4_grouped_ffn_noalloc(xc, xs, layer.x_gs, *layer.w13, *layer.w2, layer.h_gs, case.k,
                                          r.expert_offsets, r.sorted_pair_ids, r.topk_w, po, ps, sq)
        torch.cuda.synchronize()
        assert torch.equal(po, po_ref), f"{name}: pair_out differs"
        assert torch.equal(ps, ps_ref), f"{name}: pair_scale differs"
        assert torch.equal(sq, sq_ref), f"{name}: pair_sqnorm differs"
        assert bool(torch.isfinite(po).all()) and bool(torch.isfinite(ps).all())
        # and without the sums of squares
        po2 = torch.full((n, H), float("nan"), dtype=torch.float16, device="cuda")
        ps2 = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        ops.moe_nvfp4_grouped_ffn_noalloc(xc, xs, layer.x_gs, *layer.w13, *layer.w2, layer.h_gs, case.k,
                                          r.expert_offsets, r.sorted_pair_ids, r.topk_w, po2, ps2, None)
        torch.cuda.synchronize()
        assert torch.equal(po2, po_ref), f"{name}: pair_out differs without pair_sqnorm"
        assert torch.equal(ps2, ps_ref), f"{name}: pair_scale differs without pair_sqnorm"


def test_noalloc_captured_in_a_graph(ops):
    """The reason for the entry point: it can be captured in a HIP graph (no allocation, no memset
    node).  One call is captured after an eager warm-up call, then the graph is replayed three
    times, with eager work on the outputs and synchronizations between the replays.  Every replay
    must equal the workspace call bitwise."""
    case = random_case("noalloc_graph", 74, 200, 512, 256, 8, 2)
    say(f"noalloc graph: T={case.T} H={case.H} I={case.I} E={case.E} k={case.k}")
    layer = gpu_layer(case)
    r, xc, xs = ops.moe_route_quantize(dev_bf16(case.x), layer.w_router, layer.bias, case.k, case.rsf, layer.x_gs)
    n, H = case.T * case.k, case.H
    po_ref = torch.empty((n, H), dtype=torch.float16, device="cuda")
    ps_ref = torch.empty((n,), dtype=torch.float32, device="cuda")
    sq_ref = torch.empty((n,), dtype=torch.float32, device="cuda")
    ops.moe_nvfp4_grouped_ffn(xc, xs, layer.x_gs, *layer.w13, *layer.w2, layer.h_gs, case.k, r.expert_offsets,
                              r.sorted_pair_ids, r.topk_w, pair_out=po_ref, pair_scale=ps_ref, pair_sqnorm=sq_ref)
    po = torch.empty((n, H), dtype=torch.float16, device="cuda")
    ps = torch.empty((n,), dtype=torch.float32, device="cuda")
    sq = torch.empty((n,), dtype=torch.float32, device="cuda")
    args = (xc, xs, layer.x_gs, *layer.w13, *layer.w2, layer.h_gs, case.k, r.expert_offsets, r.sorted_pair_ids,
            r.topk_w, po, ps, sq)
    ops.moe_nvfp4_grouped_ffn_noalloc(*args)  # eager: the per-device set-up happens outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ops.moe_nvfp4_grouped_ffn_noalloc(*args)
    torch.cuda.synchronize()
    for rep in range(3):
        po.fill_(float("nan"))
        ps.fill_(float("nan"))
        sq.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(po, po_ref), f"replay {rep}: pair_out differs"
        assert torch.equal(ps, ps_ref), f"replay {rep}: pair_scale differs"
        assert torch.equal(sq, sq_ref), f"replay {rep}: pair_sqnorm differs"
