"""GPU parity of the BF16 shared expert and the MoE block output against
oracle/shared.py.

Tolerances: shared output and block output rel-L2 <= 2e-3 (FP32 sums of exact
BF16 products against FP64); h (BF16) rel-L2 <= 2e-3, and at least 98% of h
bitwise equal to the oracle's (h is rounded to BF16 on both sides, from FP32
here and from FP64 there, so values near a rounding midpoint may differ by one
ulp).  Both kernel families are covered: T <= 16 (split-K weight stream) and
T > 16 (LDS-tiled), with ragged tiles and a strided x.
"""

import zlib

import numpy as np
import pytest
import torch

from gpu_cases import bf16_round, check_routing, dev_bf16, gpu_layer, random_case, rel_l2, say, to_np
from oracle import moe as omoe
from oracle import shared as osh
from workloads import gen

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from nvfp4_w4a4_mixture_amd import ops as _ops

    return _ops


def _weights(seed, H, I, scale=0.02):
    rng = np.random.default_rng(seed)
    bf = lambda a: gen.f32_to_bf16_bits(np.asarray(a, np.float32))  # noqa: E731
    return bf(rng.standard_normal((I, H)) * scale), bf(rng.standard_normal((I, H)) * scale), \
        bf(rng.standard_normal((H, I)) * scale)


def _check_h(h_gpu_bits, h_ref):
    h_gpu = gen.bf16_bits_to_f32(h_gpu_bits).astype(np.float64)
    err = rel_l2(h_gpu, h_ref)
    same = float(np.mean(h_gpu == h_ref))
    print(f"  h rel-L2 {err:.3e}, bitwise equal {same:.4f}", flush=True)
    assert err <= TOL and same >= 0.98


@pytest.mark.parametrize("T,H,I,pad", [
    (1, 256, 128, 0), (5, 512, 384, 0), (16, 1024, 256, 0), (16, 768, 640, 8),  # split-K stream
    (17, 256, 128, 0), (100, 512, 256, 0), (300, 768, 384, 16), (513, 256, 256, 0),  # tiled, ragged
])
def test_shared_expert_parity(ops, T, H, I, pad):
    seed = zlib.crc32(f"{T},{H},{I},{pad}".encode())
    wg, wu, wd = _weights(seed, H, I)
    rng = np.random.default_rng(seed + 1)
    x = gen.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    xs = np.zeros((T, H + pad), np.uint16)
    xs[:, :H] = x
    x_dev = dev_bf16(xs)[:, :H]  # row stride H + pad
    w13 = dev_bf16(np.concatenate([wg, wu], axis=0))
    w2 = dev_bf16(wd)
    say(f"shared expert T={T} H={H} I={I} ldx={H + pad}")
    out = ops.moe_shared_expert(x_dev, w13, w2)
    h = ops.moe_shared_gate_up(x_dev, w13)
    out2 = ops.moe_shared_down(h, w2)
    torch.cuda.synchronize()
    ref, h_ref = osh.shared_expert(x, wg, wu, wd)
    err = rel_l2(to_np(out), ref)
    print(f"  shared rel-L2 {err:.3e}", flush=True)
    assert err <= TOL
    _check_h(to_np(h.view(torch.int16)).view(np.uint16), h_ref)
    assert torch.equal(out, out2)  # the fused call is its two stages
    again = ops.moe_shared_expert(x_dev, w13, w2)
    torch.cuda.synchronize()
    assert torch.equal(out, again)  # deterministic


def test_shared_expert_zero_tokens(ops):
    wg, wu, wd = _weights(9, 256, 128)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    out = ops.moe_shared_expert(x, dev_bf16(np.concatenate([wg, wu])), dev_bf16(wd))
    assert out.shape == (0, 256)


@pytest.mark.parametrize("name,T,H,I,E,k", [("block_small", 12, 512, 256, 16, 4), ("block_tiled", 300, 512, 256, 8, 2)])
def test_block_output_parity(ops, name, T, H, I, E, k):
    """y = routed combine + shared expert, through the layer (shared expert on its own stream)."""
    case = random_case(name, zlib.crc32(name.encode()) % 1000, T, H, I, E, k)
    wg, wu, wd = _weights(zlib.crc32(name.encode()) + 7, H, I)
    layer = gpu_layer(case)
    layer.set_shared_expert(dev_bf16(np.concatenate([wg, wu], axis=0)), dev_bf16(wd))
    say(f"block output {name}")
    x = dev_bf16(case.x)
    out = layer(x, out_dtype=torch.float32, block=True)
    torch.cuda.synchronize()
    ref = omoe.moe_layer(case.x, case.wr, case.bias, case.k, case.rsf, case.gs_x, case.experts_q, case.gs_h)
    check_routing(to_np(out.route.topk_ids), to_np(out.route.topk_w), ref, case.rsf, E, case.x, case.wr, case.bias)
    s_ref, _ = osh.shared_expert(case.x, wg, wu, wd)
    y_ref = osh.block_output(ref["y"], s_ref)
    err = rel_l2(to_np(out.y), y_ref)
    print(f"  block y rel-L2 {err:.3e}", flush=True)
    assert err <= TOL
    out16 = layer(x, out_dtype=torch.bfloat16, block=True)
    torch.cuda.synchronize()
    err16 = rel_l2(out16.y.float().cpu().numpy(), bf16_round(y_ref))
    assert err16 <= TOL
    # the routed-only output of the same layer is unchanged by the shared expert
    plain = layer(x, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert rel_l2(to_np(plain.y), ref["y"]) <= TOL
