"""GPU parity of the offline Hadamard rotation (hadamard_rotate_bf16) against
oracle/rotation.py, and the rotated outlier layer at full size.

Both sides sum the +-1 products exactly in FP64, divide once by sqrt(b) and
round once to BF16, so the rotated values are compared bitwise.  The rotated
layer is held to the layer bar (y rel-L2 <= 2e-3) against the oracle's rotated
layer on sampled tokens.  The full-size test also prints the output
error of the quantized layer, rotated and not, against the unquantized BF16
layer (a measurement, not a pass criterion).
"""

import numpy as np
import pytest
import torch

from gpu_cases import check_routing, dev_bf16, rel_l2, say, to_np
from oracle import moe as omoe
from oracle import rotation as orot
from workloads import by_name, gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from nvfp4_w4a4_mixture_amd import ops as _ops

    return _ops


def _compare_bits(got_bits, want_bits):
    same = float(np.mean(got_bits == want_bits))
    print(f"  bitwise equal {same:.6f}", flush=True)
    assert np.array_equal(got_bits, want_bits)


@pytest.mark.parametrize("rows,cols,block,pad,signed", [
    (7, 256, 2, 0, True), (33, 512, 8, 8, True), (5, 6144, 2048, 0, True), (3, 6144, 16, 0, False),
    (9, 1024, 1024, 16, True), (64, 6144, 128, 0, True), (2, 16384, 16384, 0, True), (4, 48, 16, 0, True),
    (3, 96, 32, 8, True), (6, 6144, 4, 0, True), (2, 6144, 512, 0, True),
])
def test_rotate_parity(ops, rows, cols, block, pad, signed):
    rng = np.random.default_rng(rows * 7 + cols + block)
    x = gen.f32_to_bf16_bits(rng.standard_normal((rows, cols)).astype(np.float32))
    buf = np.zeros((rows, cols + pad), np.uint16)
    buf[:, :cols] = x
    xd = dev_bf16(buf)[:, :cols]
    s = gen.rotation_signs(cols) if signed else np.ones(cols, np.float32)
    sd = torch.from_numpy(s).cuda() if signed else None
    say(f"rotate rows={rows} cols={cols} block={block} pad={pad}")
    out = ops.hadamard_rotate_bf16(xd, sd, block)
    torch.cuda.synchronize()
    want = orot.rotate_bf16(x, s, block)
    _compare_bits(to_np(out.view(torch.int16)).view(np.uint16), want)
    # in place gives the same bits
    ops.hadamard_rotate_bf16(xd, sd, block, out=xd)
    torch.cuda.synchronize()
    assert torch.equal(xd, out)


def test_rotation_keeps_routing(ops):
    """x and the router rotated by the same R: the logits are unchanged in exact arithmetic, so the top-k
    differs only where the BF16 rounding of the rotated operands moves a close decision."""
    rng = np.random.default_rng(11)
    T, H, E, k = 512, 2048, 64, 8
    x = gen.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wr = gen.f32_to_bf16_bits((rng.standard_normal((E, H)) * 0.02).astype(np.float32))
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    s = torch.from_numpy(gen.rotation_signs(H)).cuda()
    say("routing of rotated operands")
    b = torch.from_numpy(bias).cuda()
    r0 = ops.moe_route(dev_bf16(x), dev_bf16(wr), b, k, 2.5)
    r1 = ops.moe_route(ops.hadamard_rotate_bf16(dev_bf16(x), s, 2048), ops.hadamard_rotate_bf16(dev_bf16(wr), s, 2048),
                       b, k, 2.5)
    torch.cuda.synchronize()
    same = np.all(np.sort(to_np(r0.topk_ids), axis=1) == np.sort(to_np(r1.topk_ids), axis=1), axis=1)  # as sets
    # the rotated operands carry BF16 rounding (2^-9 relative per element), which moves a logit by about
    # 1e-3 and a sigmoid score by a quarter of that; tokens whose k-th and (k+1)-th scores are further apart
    # than 4e-3 keep their experts
    from oracle import routing as oroute
    _, _, _, gap = oroute.route(x, wr, bias, k, 2.5)
    clear = gap > 4e-3
    print(f"  tokens with the same top-k set: {same.mean():.4f}; with a score margin > 4e-3: {clear.mean():.4f}",
          flush=True)
    assert np.all(same[clear]) and np.array_equal(to_np(r0.topk_ids), oroute.route(x, wr, bias, k, 2.5)[0])


def test_rotated_outlier_layer_full_size(ops):
    """The 128-expert outlier layer (8192 tokens) with rotation blocks 16, 128 and 2048."""
    from nvfp4_w4a4_mixture_amd import workload_io
    from nvfp4_w4a4_mixture_amd.layer import NVFP4MoELayer

    cfg = by_name("outlier_128e")
    ws = cfg.weights
    say(f"rotated outlier layer: {cfg.describe()}")
    xb = gen.tokens(cfg)
    x = workload_io.bf16_to_device(xb, "cuda")
    wr, bias = gen.router_weight(ws), gen.router_bias(cfg)
    gs_x, gs_h = gen.global_scales(ws)
    layer, _ = workload_io.build_layer(cfg)
    base = layer(x, out_dtype=torch.float32)
    y0, ids0 = to_np(base.y), to_np(base.route.topk_ids)
    del layer, base
    signs = gen.rotation_signs(ws.H)
    sd = torch.from_numpy(signs).cuda()
    ys, idss = {}, {}
    for blk in (16, 128, 2048):
        say(f"  rotation block {blk}")
        w13, w2 = workload_io.expert_weights_bf16(ws, "cuda")
        ops.hadamard_rotate_bf16(w13.view(-1, ws.H), sd, blk, out=w13.view(-1, ws.H))
        wr_rot = ops.hadamard_rotate_bf16(dev_bf16(wr), sd, blk)
        gsx = torch.tensor([gen.rotated_gs_x(ws, blk)], dtype=torch.float32, device="cuda")
        lr = NVFP4MoELayer.from_bf16(wr_rot, torch.from_numpy(bias).cuda(), cfg.k, cfg.rsf, gsx,
                                     torch.from_numpy(gs_h).cuda(), w13, w2)
        del w13, w2
        out = lr(ops.hadamard_rotate_bf16(x, sd, blk), out_dtype=torch.float32)
        torch.cuda.synchronize()
        ys[blk], idss[blk] = to_np(out.y), to_np(out.route.topk_ids)
        if blk == 128:  # parity of the rotated layer against the oracle's, on sampled tokens
            tok = [int(t) for t in np.random.default_rng(5).choice(cfg.T, 2, replace=False)]
            xr = orot.rotate_bf16(xb[tok], signs, blk)
            wrr = orot.rotate_bf16(wr, signs, blk)
            from oracle import routing as oroute
            ids_ref, _, w64, gap = oroute.route(xr, wrr, bias, cfg.k, cfg.rsf)
            check_routing(idss[blk][tok], to_np(out.route.topk_w)[tok],
                          {"ids": ids_ref, "weights64": w64, "gap": gap}, cfg.rsf, cfg.E, xr, wrr, bias)
            need = sorted(set(int(e) for e in ids_ref.reshape(-1)))
            q = {}
            for e, g, u, d in gen.iter_experts_bf16(ws, need):
                f32 = gen.bf16_bits_to_f32
                q[e] = omoe.quantize_expert(f32(orot.rotate_bf16(g, signs, blk)), f32(orot.rotate_bf16(u, signs, blk)),
                                            f32(d))
            ref = omoe.moe_layer(xr, wrr, bias, cfg.k, cfg.rsf, gen.rotated_gs_x(ws, blk), lambda e: q[e], gs_h)
            err = rel_l2(ys[blk][tok], ref["y"])
            print(f"  rotated layer (block 128) vs oracle on tokens {tok}: rel-L2 {err:.3e}", flush=True)
            assert err <= 2e-3
        del lr, out
        torch.cuda.empty_cache()
    # measurement: error of each quantized layer against the unquantized BF16 layer, on sampled tokens whose
    # routing is the same in every variant
    rng = np.random.default_rng(9)
    cand = rng.choice(cfg.T, 64, replace=False)
    agree = [t for t in cand if all(np.array_equal(idss[b][t], ids0[t]) for b in idss)][:8]
    experts = {}
    need = sorted(set(int(e) for e in ids0[agree].reshape(-1)))
    for e, g, u, d in gen.iter_experts_bf16(ws, need):
        experts[e] = (g, u, d)
    ref = orot.moe_layer_reference(xb, wr, bias, cfg.k, cfg.rsf, lambda e: experts[e], tokens=agree)
    line = {"unrotated": rel_l2(y0[agree], ref["y"])}
    for b in ys:
        line[f"block_{b}"] = rel_l2(ys[b][agree], ref["y"])
    routing_same = {b: float(np.mean(np.all(idss[b] == ids0, axis=1))) for b in idss}
    print(f"  output error vs the unquantized layer on {len(agree)} tokens: {line}", flush=True)
    print(f"  share of tokens with the unrotated top-k: {routing_same}", flush=True)
    assert len(agree) >= 4
