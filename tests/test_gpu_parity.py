"""GPU parity: every C-ABI entry point against the CPU oracle, on seeded inputs.

Bit-exact: NVFP4 codes and scales (activations and weights), top-k ids,
expert counts/offsets and the permutation.  Tolerances: topk_w within
1e-6 * rsf, layer output rel-L2 <= 2e-3 (FP32 output against the FP64
oracle; BF16 output against the oracle rounded to BF16), REAP saliency
within 1e-3 relative.  Shapes span several tiles with ragged tails, empty
experts, a single token, k = E, E = 1, and T = 0.
"""

import json
import os
import zlib

import numpy as np
import pytest
import torch

from gpu_cases import (bf16_round, check_routing, config_case, dev_bf16, expected_pair_scale, gpu_layer, oracle_codes,
                       oracle_layer, oracle_perm, pair_rows, random_case, rel_l2, say, to_np, untile_weight_scales)
from oracle import nvfp4 as onv
from oracle import routing as oroute
from workloads import by_name, gen

pytestmark = pytest.mark.gpu

Y_TOL = 2e-3
SAL_TOL = 1e-3


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from nvfp4_w4a4_mixture_amd import ops as _ops

    return _ops


def test_library_loaded_in_tree(ops):
    path = ops.lib()._name
    assert os.path.exists(path) and "nvfp4_w4a4_mixture_amd" in path
    assert ops.lib().moe_abi_version() == 3


# ---------------------------------------------------------------------------
# quantization

def _q_case(rows, cols, dist, seed):
    rng = np.random.default_rng(seed)
    if dist == "normal":
        x = rng.standard_normal((rows, cols))
    elif dist == "wide":  # per-row magnitudes over 2^-14 .. 2^8: subnormal and saturated block scales
        x = rng.standard_normal((rows, cols)) * np.exp2(rng.uniform(-14, 8, (rows, 1)))
    elif dist == "sparse":  # zero blocks and lone values
        x = rng.standard_normal((rows, cols)) * (rng.random((rows, cols)) < 0.05)
    elif dist == "ties":  # values on E2M1 decision boundaries for gs such that inv == 1
        x = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -2.5, 6.0, -6.0], (rows, cols))
    else:
        raise ValueError(dist)
    return gen.f32_to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("rows,cols,dist,gs", [
    (1, 16, "normal", None), (333, 256, "normal", None), (64, 6144, "normal", None), (257, 512, "wide", None),
    (100, 128, "sparse", None), (40, 64, "ties", 448.0), (50, 96, "normal", 1e5), (50, 96, "normal", 1e-3)])
def test_quantize_act_bitexact(ops, rows, cols, dist, gs):
    say(f"quantize_act rows={rows} cols={cols} dist={dist} gs={gs}")
    xb = _q_case(rows, cols, dist, rows * 7 + cols)
    xf = gen.bf16_bits_to_f32(xb)
    g = np.float32(gs) if gs is not None else onv.global_scale(np.max(np.abs(xf)))
    codes_ref, scales_ref = onv.quantize(xf, g)
    codes, scales = ops.nvfp4_quantize_act(dev_bf16(xb), torch.tensor([g], dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(to_np(scales), scales_ref)
    assert np.array_equal(to_np(codes), onv.pack_codes(codes_ref))


def test_quantize_act_with_leading_dimension(ops):
    say("quantize_act ld > cols")
    xb = _q_case(70, 384, "normal", 5)
    full = dev_bf16(xb)
    sub = full[:, 128:384]  # ld = 384, cols = 256, 16-byte aligned start
    g = np.float32(300.0)
    codes, scales = ops.nvfp4_quantize_act(sub, torch.tensor([g], dtype=torch.float32, device="cuda"))
    c_ref, s_ref = onv.quantize(gen.bf16_bits_to_f32(xb[:, 128:384]), g)
    assert np.array_equal(to_np(scales), s_ref)
    assert np.array_equal(to_np(codes), onv.pack_codes(c_ref))


def test_quantize_act_golden_blocks(ops, golden_dir):
    with open(os.path.join(golden_dir, "nvfp4_blocks.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        say(f"golden block {case['name']}")
        xb = gen.f32_to_bf16_bits(np.array([case["x"]], np.float32))
        g = np.float32(case["gs"])
        codes, scales = ops.nvfp4_quantize_act(dev_bf16(xb), torch.tensor([g], dtype=torch.float32, device="cuda"))
        assert int(to_np(scales)[0, 0]) == int(case["scale"], 16), case["name"]
        assert to_np(codes)[0].tolist() == [int(b, 16) for b in case["packed"]], case["name"]


def test_quantize_weights_bitexact(ops):
    say("quantize_weights batch=3 (one all-zero matrix)")
    rng = np.random.default_rng(3)
    w = rng.standard_normal((3, 48, 256)).astype(np.float32) * np.array([0.02, 0.0, 0.3], np.float32)[:, None, None]
    w[2, 5, 7] = 1.5  # a lone outlier sets the third matrix's global scale
    wb = gen.f32_to_bf16_bits(w)
    codes, scales, gs = ops.nvfp4_quantize_weights(dev_bf16(wb))
    torch.cuda.synchronize()
    for b in range(3):
        c_ref, s_ref, g_ref = onv.quantize_weight(gen.bf16_bits_to_f32(wb[b]))
        assert to_np(gs)[b] == g_ref
        assert np.array_equal(untile_weight_scales(to_np(scales))[b], s_ref)
        assert np.array_equal(to_np(codes)[b], c_ref)
    assert to_np(gs)[1] == 1.0


# ---------------------------------------------------------------------------
# routing + permutation

# Logits: FP64 MFMA kernel when rows are 16-byte aligned and H % 16 == 0 (H-split across waves for T <= 16,
# E <= 128), else the vector kernels (H = 520: register/LDS decode kernel; E = 256 at T = 16: same).
# Permutation: one workgroup up to 16 tokens, else the chunked counting sort.
@pytest.mark.parametrize("T,H,E,k", [(64, 256, 8, 2), (300, 512, 80, 8), (1000, 256, 128, 8), (37, 64, 256, 16),
                                     (5, 32, 1, 1), (3, 32, 16, 16), (2500, 128, 80, 8), (0, 64, 8, 2),
                                     (64, 64, 128, 16), (16, 6144, 80, 8), (16, 6144, 256, 256), (13, 520, 200, 9)])
def test_route_and_permutation_bitexact(ops, T, H, E, k):
    say(f"route T={T} H={H} E={E} k={k}")
    rng = np.random.default_rng(T * 31 + E)
    xb = gen.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wr = gen.f32_to_bf16_bits((rng.standard_normal((E, H)) * 0.05).astype(np.float32))
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    rsf = 2.5
    out = ops.moe_route(dev_bf16(xb), dev_bf16(wr), torch.from_numpy(bias).cuda(), k, rsf)
    torch.cuda.synchronize()
    counts, offsets, perm = to_np(out.expert_counts), to_np(out.expert_offsets), to_np(out.sorted_pair_ids)
    if T == 0:
        assert counts.tolist() == [0] * E and offsets.tolist() == [0] * (E + 1)
        return
    ids, w = to_np(out.topk_ids), to_np(out.topk_w)
    ref = dict(zip(("ids", "weights", "weights64", "gap"), oroute.route(xb, wr, bias, k, rsf)))
    check_routing(ids, w, ref, rsf, E, xb, wr, bias)
    c_ref, o_ref, p_ref = oracle_perm(ids, E)
    assert np.array_equal(counts, c_ref)
    assert np.array_equal(offsets, o_ref)
    assert np.array_equal(perm, p_ref)


@pytest.mark.parametrize("T,H,pad", [(10, 256, 4), (10, 256, 8), (16, 1024, 24)])
def test_route_strided_rows(ops, T, H, pad):
    """x as a column slice of a wider buffer: ldx % 8 != 0 takes the general path at decode sizes."""
    say(f"route strided T={T} H={H} ldx={H + pad}")
    E, k, rsf = 40, 6, 1.5
    rng = np.random.default_rng(T + pad)
    xw = gen.f32_to_bf16_bits(rng.standard_normal((T, H + pad)).astype(np.float32))
    wr = gen.f32_to_bf16_bits((rng.standard_normal((E, H)) * 0.05).astype(np.float32))
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    x = dev_bf16(xw)[:, :H]
    assert x.stride(0) == H + pad
    out = ops.moe_route(x, dev_bf16(wr), torch.from_numpy(bias).cuda(), k, rsf)
    torch.cuda.synchronize()
    xb = np.ascontiguousarray(xw[:, :H])
    ref = dict(zip(("ids", "weights", "weights64", "gap"), oroute.route(xb, wr, bias, k, rsf)))
    ids = to_np(out.topk_ids)
    check_routing(ids, to_np(out.topk_w), ref, rsf, E, xb, wr, bias)
    c_ref, o_ref, p_ref = oracle_perm(ids, E)
    assert np.array_equal(to_np(out.expert_counts), c_ref)
    assert np.array_equal(to_np(out.expert_offsets), o_ref)
    assert np.array_equal(to_np(out.sorted_pair_ids), p_ref)


@pytest.mark.parametrize("T,H,E,k", [(16, 6144, 80, 8), (300, 512, 80, 8), (16, 1024, 256, 8), (1, 256, 8, 2),
                                     (70, 768, 128, 4)])
# (16, 1024, 256, 8): decode batch with E > 128 takes the register/LDS logits kernel and a separate quantize pass
def test_route_quantize_matches_route_and_quantize(ops, T, H, E, k):
    say(f"route_quantize T={T} H={H} E={E} k={k}")
    rng = np.random.default_rng(T * 7 + H + E)
    xb = gen.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wr = gen.f32_to_bf16_bits((rng.standard_normal((E, H)) * 0.05).astype(np.float32))
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    g = float(np.float32(2688.0 / np.abs(gen.bf16_bits_to_f32(xb)).max()))
    gs = torch.tensor([g], dtype=torch.float32, device="cuda")
    out, codes, scales = ops.moe_route_quantize(dev_bf16(xb), dev_bf16(wr), torch.from_numpy(bias).cuda(), k, 2.5, gs)
    torch.cuda.synchronize()
    c_ref, s_ref = onv.quantize(gen.bf16_bits_to_f32(xb), np.float32(g))
    assert np.array_equal(to_np(codes), onv.pack_codes(c_ref))
    assert np.array_equal(to_np(scales), s_ref)
    ids = to_np(out.topk_ids)
    ref = dict(zip(("ids", "weights", "weights64", "gap"), oroute.route(xb, wr, bias, k, 2.5)))
    check_routing(ids, to_np(out.topk_w), ref, 2.5, E, xb, wr, bias)
    c_ref, o_ref, p_ref = oracle_perm(ids, E)
    assert np.array_equal(to_np(out.expert_counts), c_ref)
    assert np.array_equal(to_np(out.expert_offsets), o_ref)
    assert np.array_equal(to_np(out.sorted_pair_ids), p_ref)


@pytest.mark.parametrize("T", [12, 40, 200])  # decode path, general path (one and several chunks)
def test_route_exact_ties_go_to_lower_index(ops, T):
    say(f"route crafted ties T={T}")
    H, E, k = 64, 12, 4
    rng = np.random.default_rng(8)
    wr = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    wr[5] = wr[2]
    wr[9] = wr[2]
    wr[7] = wr[3]
    wrb = gen.f32_to_bf16_bits(wr)
    bias = np.zeros(E, np.float32)
    bias[2] = bias[5] = bias[9] = 2.0  # score > 2 > any other: tied experts 2, 5, 9 lead every token
    xb = gen.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    out = ops.moe_route(dev_bf16(xb), dev_bf16(wrb), torch.from_numpy(bias).cuda(), k, 1.0)
    ids = to_np(out.topk_ids)
    ref_ids, w32_ref, w64_ref, gap = oroute.route(xb, wrb, bias, k, 1.0)
    assert np.array_equal(ids, ref_ids)
    # every token has an exact tie inside its top-k: validated as near-tie tokens too
    check_routing(ids, to_np(out.topk_w), {"ids": ref_ids, "weights64": w64_ref, "gap": gap}, 1.0, E, xb, wrb, bias)
    assert np.all(ids[:, :3] == [2, 5, 9])


@pytest.mark.parametrize("T,H,E,k,nan_bias", [(12, 256, 40, 6, False), (300, 512, 80, 8, True), (40, 64, 16, 16, False)])
def test_route_nonfinite_inputs(ops, T, H, E, k, nan_bias):
    """Tokens whose x holds a NaN or infinities (so their logits are NaN or infinite), and NaN
    biases: the selection ranks NaN scores below every number, so ids and the permutation still
    equal the oracle's (a stable descending sort, NaN last) and every slot is written."""
    say(f"route nonfinite T={T} H={H} E={E} k={k} nan_bias={nan_bias}")
    rng = np.random.default_rng(T + E)
    xf = rng.standard_normal((T, H)).astype(np.float32)
    xf[3, 7] = np.nan  # every logit of token 3 is NaN
    xf[5, 11] = np.inf  # token 5: +-inf (or NaN where the router weight is 0)
    xf[8, 2], xf[8, 9] = np.inf, -np.inf  # token 8: mixed
    if T == 40:
        xf[:] = np.nan  # every token NaN: ids 0..k-1 in order
    xb = gen.f32_to_bf16_bits(np.where(np.isfinite(xf), xf, 0)).astype(np.uint16)
    special = ~np.isfinite(xf)
    xb[special] = np.where(np.isnan(xf[special]), 0x7FC0, np.where(xf[special] > 0, 0x7F80, 0xFF80)).astype(np.uint16)
    wr = gen.f32_to_bf16_bits((rng.standard_normal((E, H)) * 0.05).astype(np.float32))
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    if nan_bias:
        bias[[4, 17]] = np.nan
    ids_ref, _, w64_ref, _ = oroute.route(xb, wr, bias, k, 2.5)
    out = ops.moe_route(dev_bf16(xb), dev_bf16(wr), torch.from_numpy(bias).cuda(), k, 2.5)
    torch.cuda.synchronize()
    ids, w = to_np(out.topk_ids), to_np(out.topk_w).astype(np.float64)
    assert np.array_equal(ids, ids_ref)
    assert np.array_equal(np.isnan(w), np.isnan(w64_ref))
    fin = ~np.isnan(w64_ref)
    assert np.all(np.abs(w[fin] - w64_ref[fin]) <= 1e-6 * 2.5)
    c_ref, o_ref, p_ref = oracle_perm(ids_ref, E)
    assert np.array_equal(to_np(out.expert_counts), c_ref)
    assert np.array_equal(to_np(out.expert_offsets), o_ref)
    assert np.array_equal(to_np(out.sorted_pair_ids), p_ref)
    if T == 40:
        assert np.all(ids == np.arange(k))


# ---------------------------------------------------------------------------
# whole layer

def _layer_check(ops, case, reap=True):
    say(f"layer {case.name}: T={case.T} H={case.H} I={case.I} E={case.E} k={case.k}")
    layer = gpu_layer(case)
    # weights: GPU RTN == oracle RTN, bitwise
    c13, s13, g13 = (to_np(t) for t in layer.w13)
    c2, s2, g2 = (to_np(t) for t in layer.w2)
    s13, s2 = untile_weight_scales(s13), untile_weight_scales(s2)
    for e, q in enumerate(case.experts_q):
        assert np.array_equal(c13[e, :case.I], q.gate_codes) and np.array_equal(c13[e, case.I:], q.up_codes)
        assert np.array_equal(s13[e, :case.I], q.gate_scales) and np.array_equal(s13[e, case.I:], q.up_scales)
        assert np.array_equal(c2[e], q.down_codes) and np.array_equal(s2[e], q.down_scales)
        assert g13[e, 0] == q.gate_gs and g13[e, 1] == q.up_gs and g2[e] == q.down_gs
    x = dev_bf16(case.x)
    out32 = layer(x, out_dtype=torch.float32, reap=reap)
    torch.cuda.synchronize()
    ref = oracle_layer(case, with_pairs=True)
    ids, w = to_np(out32.route.topk_ids), to_np(out32.route.topk_w)
    check_routing(ids, w, ref, case.rsf, case.E, case.x, case.wr, case.bias)
    c_ref, s_ref = oracle_codes(case)
    assert np.array_equal(to_np(out32.x_codes), c_ref) and np.array_equal(to_np(out32.x_scales), s_ref)
    y32 = to_np(out32.y)
    err = rel_l2(y32, ref["y"])
    pair_ref = ref["pair_f"] * ref["weights64"].reshape(-1)[:, None]
    perr = rel_l2(pair_rows(out32.pair_out, out32.pair_scale), pair_ref)
    print(f"  rel-L2 y(fp32)={err:.3e} pair rows={perr:.3e}", flush=True)
    assert err <= Y_TOL and perr <= Y_TOL
    # the row scales follow the stated rule exactly; the FP16 values stay below 2^15
    ps = to_np(out32.pair_scale)
    assert np.array_equal(ps, expected_pair_scale(w, ids, case.I, to_np(layer.h_gs), to_np(layer.w2[2])))
    assert float(out32.pair_out.abs().max()) < 2.0 ** 15
    # and they are rounded to nearest: within half an FP16 ulp of the oracle's value over the row scale, up to the
    # FP32-against-FP64 difference of f (1e-5 relative); a truncating or double-rounding encoder would miss about
    # half the elements.  Rows whose h codes sit on the other side of a rounding boundary (rare) are in the 1%.
    ref_s = pair_ref / ps.astype(np.float64)[:, None]
    got_s = to_np(out32.pair_out).astype(np.float64)
    e2 = np.floor(np.log2(np.maximum(np.abs(ref_s), 2.0 ** -24))).astype(np.int64)  # binade of the value
    ulp = np.ldexp(1.0, np.maximum(e2, -14) - 10)
    rounded = np.abs(got_s - ref_s) <= 0.5 * ulp + 1e-5 * np.abs(ref_s)
    print(f"  pair values within half an FP16 ulp: {rounded.mean():.6f}", flush=True)
    assert rounded.mean() >= 0.99
    if reap:
        sal = to_np(out32.saliency).astype(np.float64)
        cnt = np.bincount(ids.reshape(-1), minlength=case.E)
        nz = cnt > 0
        rel = np.abs(sal[nz] - ref["saliency"][nz]) / ref["saliency"][nz]
        print(f"  saliency max rel={rel.max():.3e}", flush=True)
        assert rel.max() <= SAL_TOL
        assert np.all(sal[~nz] == 0.0)
        sq = to_np(out32.pair_sqnorm).astype(np.float64)
        assert rel_l2(np.sqrt(sq), ref["pair_norm"]) <= Y_TOL
    y16 = layer(x, out_dtype=torch.bfloat16, reap=False)
    torch.cuda.synchronize()
    err16 = rel_l2(y16.y.float().cpu().numpy(), bf16_round(ref["y"]))
    print(f"  rel-L2 y(bf16 vs bf16(ref))={err16:.3e}", flush=True)
    assert err16 <= Y_TOL
    return layer, out32, ref


def test_layer_parity_config0(ops):
    _layer_check(ops, config_case(by_name("tiny")))


@pytest.mark.parametrize("name,T,H,I,E,k", [
    ("ragged_tiles", 300, 512, 256, 8, 2),
    ("multi_mtile", 300, 256, 128, 3, 2),
    ("decode_small", 16, 512, 256, 16, 4),
    ("single_token", 1, 256, 128, 8, 2),
    ("dense_e1_k1", 20, 256, 128, 1, 1),
    ("k_equals_e", 17, 256, 128, 4, 4),
    ("many_empty_experts", 40, 256, 128, 256, 8),
    ("tiled_mid", 130, 768, 384, 6, 3),
    ("tiled_k5", 40, 512, 640, 4, 2),  # down K = 640: five ring stages (one past the ring depth)
    # one expert, k = 1: its m-tiles hold exactly T rows.  A last m-tile of <= 128 rows runs wide
    # (128 rows x two n-tiles) when the n-tile count is even (here 2 for both stages)
    ("e1_rows128_wide", 128, 512, 256, 1, 1),
    ("e1_rows129_full", 129, 512, 256, 1, 1),
    ("e1_rows384_full_then_wide", 384, 512, 256, 1, 1),
    # a last m-tile of <= 64 rows runs as the half tile (64 rows x two n-tiles); 65 rows stays wide
    ("e1_rows64_half", 64, 512, 256, 1, 1),
    ("e1_rows17_half", 17, 512, 256, 1, 1),
    ("e1_rows65_wide", 65, 512, 256, 1, 1),
    ("e1_rows320_full_then_half", 320, 512, 256, 1, 1),
    ("many_small_half", 60, 512, 256, 32, 4),
    # decode kernel (T <= 16): four waves take 256-k iterations in turn through two register buffers
    ("stream_decode", 12, 2048, 2048, 8, 2),  # 8 iterations: two per wave in both stages
    ("stream_three_steps", 5, 3072, 2048, 6, 3),  # gate_up: 12 iterations, three per wave (ends in the first buffer)
    ("decode_uneven_waves", 10, 1280, 384, 8, 2),  # gate_up: 5 iterations (2, 1, 1, 1); down: K 384, 128-k steps
    # 8 n-tiles in both stages (I 1024, H 2048): the XCD-aware tile order, with full, ragged and wide m-tiles
    ("xcd_tiles", 600, 2048, 1024, 5, 2),
    ("xcd_tiles_wide", 250, 2048, 1024, 4, 2),
    ("xcd_tiles_half", 120, 2048, 1024, 5, 2),
    # k = 16: the combine sums each token's rows in two chunks of eight
    ("k16_decode", 9, 256, 128, 32, 16),
    ("k16_tiled", 150, 512, 256, 32, 16),
    # 256 experts at decode size: the register/LDS logits kernel (more than 128 experts), 16 of 256 chosen
    ("decode_e256_k16", 16, 256, 128, 256, 16),
])
def test_layer_parity_random(ops, name, T, H, I, E, k):
    case = random_case(name, zlib.crc32(name.encode()) % 1000, T, H, I, E, k)
    _layer_check(ops, case)


@pytest.mark.parametrize("T", [300, 9])  # tiled path, small-M path
def test_layer_parity_subnormal_weight_scales(ops, T):
    """A quarter of the weight rows shrunk by 2^-10..2^-14: their E4M3 block
    scales are subnormal and must decode exactly in the FFN."""
    case = random_case(f"subnormal_scales_{T}", 31, T, 256, 128, 6, 2, tiny_rows=0.25)
    subn = sum(int(np.sum(q.gate_scales < 8)) for q in case.experts_q)
    assert subn > 0
    _layer_check(ops, case)


@pytest.mark.parametrize("name,T,xscale,wscale", [
    ("large_outputs", 40, 1.0, 2.0),  # pair rows up to about 9e4: past FP16's largest finite value
    ("large_outputs_decode", 9, 1.0, 2.0),
    ("tiny_outputs", 40, 1e-4, 0.02),  # pair rows about 1e-9: below FP16's smallest subnormal
    ("tiny_outputs_decode", 9, 1e-4, 0.02),
])
def test_layer_parity_output_range(ops, name, T, xscale, wscale):
    """Pair rows are FP16 times a power-of-two row scale: outputs far outside FP16's own range keep full precision."""
    case = random_case(name, 5, T, 256, 128, 8, 2, xscale=xscale, wscale=wscale)
    ref = oracle_layer(case, with_pairs=True)
    peak = float(np.abs(ref["pair_f"] * ref["weights64"].reshape(-1)[:, None]).max())
    assert peak > 65504.0 if wscale > 1 else peak < 2.0 ** -24
    _layer_check(ops, case)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_combine_decodes_scaled_fp16_rows(ops, out_dtype):
    """y = sum over j, in j order, of FP16 value times its row scale, in FP32: bit for bit against numpy, for FP16
    values across their whole finite range and scales from 2^-100 to 2^100; the block combine adds the shared
    row last."""
    rng = np.random.default_rng(3)
    T, k, H = 37, 5, 264
    bits = rng.integers(0, 1 << 16, (T * k, H), dtype=np.uint16)
    bits[(bits & 0x7C00) == 0x7C00] &= 0xBFFF  # no inf or NaN: clear the top exponent bit
    vals = bits.view(np.float16)
    scale = np.ldexp(np.float32(1.0), rng.integers(-100, 101, T * k)).astype(np.float32)
    # a third of the tokens: every row at one scale, so that sums cancel and round
    same = rng.random(T) < 0.33
    scale.reshape(T, k)[same] = np.float32(2.0 ** 7)
    shared = (rng.standard_normal((T, H)) * 1e3).astype(np.float32)
    d = vals.astype(np.float32) * scale[:, None]  # exact
    y = d.reshape(T, k, H)[:, 0].copy()
    for j in range(1, k):
        y = (y + d.reshape(T, k, H)[:, j]).astype(np.float32)
    yb = (y + shared).astype(np.float32)
    po = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.float16)
    ps = torch.from_numpy(scale).cuda()
    say(f"combine of scaled FP16 rows, {out_dtype}")
    got = ops.moe_combine(po, ps, T, k, out_dtype)
    got_b = ops.moe_combine_block(po, ps, torch.from_numpy(shared).cuda(), T, k, out_dtype)
    torch.cuda.synchronize()
    if out_dtype == torch.float32:
        assert np.array_equal(to_np(got).view(np.uint32), y.view(np.uint32))
        assert np.array_equal(to_np(got_b).view(np.uint32), yb.view(np.uint32))
    else:
        assert np.array_equal(to_np(got.view(torch.int16)).view(np.uint16), gen.f32_to_bf16_bits(y))
        assert np.array_equal(to_np(got_b.view(torch.int16)).view(np.uint16), gen.f32_to_bf16_bits(yb))


def test_single_expert_output_is_rsf_times_mlp(ops):
    case = random_case("e1", 11, 24, 256, 128, 1, 1)
    layer, out, ref = _layer_check(ops, case, reap=False)
    assert np.all(to_np(out.route.topk_w) == np.float32(case.rsf))


@pytest.mark.parametrize("T", [150, 12])  # tiled path, small-M path
def test_grouped_ffn_matches_stage_calls(ops, T):
    case = random_case(f"stages{T}", 5, T, 256, 128, 5, 2)
    say(f"grouped ffn vs stage entry points T={T}")
    layer = gpu_layer(case)
    x = dev_bf16(case.x)
    out = layer(x, out_dtype=torch.float32, reap=True)  # the layer calls the two stage entry points
    r = out.route
    pair_out, pair_scale, sq = ops.moe_nvfp4_grouped_ffn(out.x_codes, out.x_scales, layer.x_gs, *layer.w13,
                                                         *layer.w2, layer.h_gs, case.k, r.expert_offsets,
                                                         r.sorted_pair_ids, r.topk_w, pair_sqnorm=True)
    torch.cuda.synchronize()
    assert torch.equal(pair_out, out.pair_out) and torch.equal(pair_scale, out.pair_scale)
    assert torch.equal(sq, out.pair_sqnorm)


def test_zero_tokens_is_a_noop(ops):
    say("T = 0")
    case = random_case("t0", 2, 4, 256, 128, 4, 2)
    layer = gpu_layer(case)
    x = torch.empty((0, case.H), dtype=torch.bfloat16, device="cuda")
    out = layer(x, out_dtype=torch.float32, reap=True)
    torch.cuda.synchronize()
    assert out.y.shape == (0, case.H)
    assert torch.all(out.route.expert_counts == 0)
    assert torch.all(out.saliency == 0)


@pytest.mark.parametrize("name,T,H,I,E,k", [
    ("det_decode", 12, 512, 256, 16, 4),       # small-M kernels, single-workgroup permutation
    ("det_tiled", 200, 256, 128, 8, 2),        # tiled kernels, ragged m-tiles
    ("det_xcd_wide", 250, 2048, 1024, 4, 2),   # XCD-aware tile order with wide half-empty m-tiles
])
def test_repeat_runs_are_bitwise_identical(ops, name, T, H, I, E, k):
    """Every reduction has a fixed order, so three runs of the same layer on the same input agree bit for bit in
    every output: routing, codes, pair rows, norms, y and the saliency."""
    case = random_case(name, 9, T, H, I, E, k)
    say(f"determinism {name}")
    layer = gpu_layer(case)
    x = dev_bf16(case.x)

    def snap(o):
        return [o.y, o.saliency, o.route.topk_ids, o.route.topk_w, o.route.expert_offsets, o.route.sorted_pair_ids,
                o.x_codes, o.x_scales, o.h_codes, o.h_scales, o.pair_out, o.pair_scale, o.pair_sqnorm]

    first = [t.clone() for t in snap(layer(x, out_dtype=torch.float32, reap=True))]
    for _ in range(2):
        again = snap(layer(x, out_dtype=torch.float32, reap=True))
        torch.cuda.synchronize()
        for i, (u, v) in enumerate(zip(first, again)):
            assert torch.equal(u, v), f"{name}: output {i} differs between runs"


def test_prepack_roundtrip_and_canonical_weights(ops):
    """unpack(prepack(w)) == w for arbitrary bytes; prepacking the oracle's canonical RTN weights gives the
    library quantizer's layout bit for bit, and a layer built from them gives the same output."""
    rng = np.random.default_rng(21)
    codes = torch.from_numpy(rng.integers(0, 256, (3, 32, 128), dtype=np.uint8)).cuda()
    scales = torch.from_numpy(rng.integers(0, 256, (3, 32, 16), dtype=np.uint8)).cuda()
    say("prepack round trip")
    pc, ps = ops.moe_nvfp4_prepack_weights(codes, scales, 1)
    uc, us = ops.moe_nvfp4_unpack_weights(pc, ps, 1)
    torch.cuda.synchronize()
    assert torch.equal(pc, codes) and torch.equal(uc, codes) and torch.equal(us, scales)
    assert np.array_equal(untile_weight_scales(to_np(ps)), to_np(scales))

    case = random_case("prepack", 23, 40, 512, 256, 6, 2)
    layer = gpu_layer(case)
    q = case.experts_q
    c13 = np.stack([np.concatenate([e.gate_codes, e.up_codes]) for e in q])
    s13 = np.stack([np.concatenate([e.gate_scales, e.up_scales]) for e in q])
    c2 = np.stack([e.down_codes for e in q])
    s2 = np.stack([e.down_scales for e in q])
    say("prepack of oracle weights")
    p13 = ops.moe_nvfp4_prepack_weights(torch.from_numpy(c13).cuda(), torch.from_numpy(s13).cuda(), 0)
    p2 = ops.moe_nvfp4_prepack_weights(torch.from_numpy(c2).cuda(), torch.from_numpy(s2).cuda(), 1)
    torch.cuda.synchronize()
    assert torch.equal(p13[0], layer.w13[0]) and torch.equal(p13[1], layer.w13[1])
    assert torch.equal(p2[0], layer.w2[0]) and torch.equal(p2[1], layer.w2[1])
    from nvfp4_w4a4_mixture_amd.layer import NVFP4MoELayer
    g13 = torch.tensor([[e.gate_gs, e.up_gs] for e in q], dtype=torch.float32, device="cuda")
    g2 = torch.tensor([e.down_gs for e in q], dtype=torch.float32, device="cuda")
    other = NVFP4MoELayer(layer.w_router, layer.bias, case.k, case.rsf, layer.x_gs, layer.h_gs, p13[0], p13[1], g13,
                          p2[0], p2[1], g2)
    x = dev_bf16(case.x)
    y0 = layer(x, out_dtype=torch.float32).y.clone()
    y1 = other(x, out_dtype=torch.float32).y
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("T", [12, 300])
def test_combine_reap_equals_separate_calls(ops, T):
    case = random_case(f"combine_reap_{T}", 41, T, 512, 256, 16, 4)
    layer = gpu_layer(case)
    say(f"combine + reap fused vs separate, T={T}")
    out = layer(dev_bf16(case.x), out_dtype=torch.bfloat16, reap=True)  # the layer's fused launch
    r = out.route
    y2 = ops.moe_combine(out.pair_out, out.pair_scale, T, case.k, torch.bfloat16)
    s2 = ops.reap_saliency(out.pair_sqnorm, r.topk_w, r.expert_offsets, r.sorted_pair_ids, T, case.k, case.E)
    torch.cuda.synchronize()
    assert torch.equal(out.y, y2) and torch.equal(out.saliency, s2)
    # no tokens: zero saliencies, nothing else written
    e = torch.full((case.E,), 7.0, device="cuda")
    off = torch.zeros((case.E + 1,), dtype=torch.int32, device="cuda")
    empty = torch.empty((0, 512), dtype=torch.float16, device="cuda")
    no_scales = torch.empty((0,), dtype=torch.float32, device="cuda")
    ops.moe_combine_reap(empty, no_scales, 0, case.k, None, None, off, None, case.E, saliency=e)
    torch.cuda.synchronize()
    assert torch.all(e == 0)
