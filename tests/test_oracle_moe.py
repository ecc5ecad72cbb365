"""Pins for the oracle's expert FFN, combine, REAP saliency and calibration (CPU).

* a pure-Python loop brute force of the whole layer on a tiny shape;
* the single-expert special case (y = rsf * dense SwiGLU MLP);
* the lossless case: operands built exactly representable in NVFP4, so the
  gate/up stage equals a plain float64 SwiGLU on those known values;
* REAP by brute-force loop and a closed form;
* calibration scales from their definition.
"""

import math

import numpy as np
import pytest

from oracle import formats, moe, nvfp4, routing
from workloads import gen


def _bf16(a):
    return gen.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _rand_layer(seed, T, H, I, E, scale=0.05):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal((T, H)))
    wr = _bf16(rng.standard_normal((E, H)) * 0.1)
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    experts = []
    for _ in range(E):
        g = gen.bf16_bits_to_f32(_bf16(rng.standard_normal((I, H)) * scale))
        u = gen.bf16_bits_to_f32(_bf16(rng.standard_normal((I, H)) * scale))
        d = gen.bf16_bits_to_f32(_bf16(rng.standard_normal((H, I)) * scale))
        experts.append(moe.quantize_expert(g, u, d))
    gs_x, gs_h = moe.calibrate(_bf16(rng.standard_normal((32, H))), experts, E)
    return x, wr, bias, experts, gs_x, gs_h


def _loop_layer(x_bf16, wr, bias, experts, gs_x, gs_h, k, rsf):
    """Brute force with Python loops and math.fsum; quantization via the pinned quantizer."""
    T, H = x_bf16.shape
    E = wr.shape[0]
    xf = gen.bf16_bits_to_f32(x_bf16)
    wrf = gen.bf16_bits_to_f32(wr)
    y = [[0.0] * H for _ in range(T)]
    for t in range(T):
        logit = [math.fsum(float(xf[t, h]) * float(wrf[e, h]) for h in range(H)) for e in range(E)]
        s = [1.0 / (1.0 + math.exp(-z)) for z in logit]
        score = [s[e] + float(bias[e]) for e in range(E)]
        chosen = sorted(range(E), key=lambda e: (-score[e], e))[:k]
        tot = sum(s[e] for e in chosen)
        xc, xs = nvfp4.quantize(xf[t:t + 1], gs_x)
        xhat = nvfp4.dequantize(xc, xs, gs_x)[0]
        for e in chosen:
            wgt = rsf * s[e] / tot
            W = experts[e]
            wg = nvfp4.dequantize_packed(W.gate_codes, W.gate_scales, W.gate_gs)
            wu = nvfp4.dequantize_packed(W.up_codes, W.up_scales, W.up_gs)
            wd = nvfp4.dequantize_packed(W.down_codes, W.down_scales, W.down_gs)
            I = wg.shape[0]
            h = []
            for i in range(I):
                g = math.fsum(xhat[c] * wg[i, c] for c in range(H))
                u = math.fsum(xhat[c] * wu[i, c] for c in range(H))
                h.append(float(np.float32(g / (1.0 + math.exp(-g)) * u)))
            hc, hs = nvfp4.quantize(np.array([h], np.float32), gs_h[e])
            hhat = nvfp4.dequantize(hc, hs, gs_h[e])[0]
            for o in range(H):
                f = math.fsum(hhat[i] * wd[o, i] for i in range(I))
                y[t][o] += wgt * f
    return np.array(y)


def test_layer_matches_loop_brute_force():
    T, H, I, E, k = 3, 32, 16, 3, 2
    x, wr, bias, experts, gs_x, gs_h = _rand_layer(5, T, H, I, E)
    out = moe.moe_layer(x, wr, bias, k, 2.5, gs_x, experts, gs_h)
    ref = _loop_layer(x, wr, bias, experts, gs_x, gs_h, k, 2.5)
    assert np.max(np.abs(out["y"] - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_single_expert_is_rsf_times_dense_mlp():
    """E = 1, k = 1: the routing weight is exactly rsf, so y = rsf * f(x)."""
    T, H, I = 5, 64, 32
    x, wr, bias, experts, gs_x, gs_h = _rand_layer(9, T, H, I, 1)
    out = moe.moe_layer(x, wr, bias, 1, 2.5, gs_x, experts, gs_h, with_pairs=True)
    assert np.all(out["ids"] == 0)
    assert np.all(out["weights64"] == 2.5)
    assert np.array_equal(out["y"], 2.5 * out["pair_f"])


def test_lossless_operands_give_plain_swiglu():
    """x and weights built from E2M1 x E4M3 values are reproduced exactly by the
    quantizer, so h equals f32(silu(x W_g^T) * (x W_u^T)) computed from the known
    values; with power-of-two global scales nothing is rounded before the matmuls."""
    rng = np.random.default_rng(21)
    T, H, I = 4, 64, 32

    def representable(rows, cols, scale_lo, scale_hi):
        nb = cols // 16
        sc = rng.integers(scale_lo, scale_hi, (rows, nb)).astype(np.uint8)
        codes = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
        codes[:, ::16] = 7
        return (formats.E2M1_VALUES[codes].reshape(rows, nb, 16) * formats.E4M3_VALUES[sc][:, :, None]).reshape(rows, cols)

    # x: block scales in [2^-3, 2); one block holding only the amax 42 makes
    # gs_x = 2688 / 42 = 64, a power of two, so every block scale is S * 64 exactly.
    x = representable(T, H, 0x20, 0x40)
    x[0, :16] = 0.0
    x[0, 0] = 6 * 448.0 / 64  # amax = 42 -> gs_x = 64
    gs_x = nvfp4.global_scale(np.max(np.abs(x)))
    assert gs_x == np.float32(64.0)
    x_bf16 = _bf16(x)
    assert np.array_equal(gen.bf16_bits_to_f32(x_bf16).astype(np.float64), x)

    def with_pow2_gs(w):
        # values c * S / 4096; one block holding only the amax 2688 / 4096 makes
        # gs = 4096, so every block scale is S exactly and dequantization is exact
        w = w / 4096.0
        w[0, :16] = 0.0
        w[0, 0] = 2688.0 / 4096.0
        return w

    wg = with_pow2_gs(representable(I, H, 0x30, 0x60))
    wu = with_pow2_gs(representable(I, H, 0x30, 0x60))
    wd = with_pow2_gs(representable(H, I, 0x30, 0x60))
    ex = moe.quantize_expert(wg.astype(np.float32), wu.astype(np.float32), wd.astype(np.float32))
    assert ex.gate_gs == ex.up_gs == ex.down_gs == np.float32(4096.0)
    dg, du, dd = ex.dequantized()
    assert np.array_equal(dg, wg) and np.array_equal(du, wu) and np.array_equal(dd, wd)

    xc, xs = nvfp4.quantize(gen.bf16_bits_to_f32(x_bf16), gs_x)
    xhat = nvfp4.dequantize(xc, xs, gs_x)
    assert np.array_equal(xhat, x)  # value(code) * (S * 64) / 64 = x

    h = moe.expert_hidden(xhat, dg, du)
    assert h.dtype == np.float32  # h is rounded once to float32 before re-quantization
    # independent statement of SwiGLU on the known values: gate rows first, then up
    for t in range(T):
        for i in range(I):
            g = math.fsum(x[t] * wg[i])
            u = math.fsum(x[t] * wu[i])
            want = np.float32(g * u / (1.0 + math.exp(-g)))
            assert abs(float(h[t, i]) - float(want)) <= float(np.spacing(np.abs(want)))


def test_reap_brute_force_and_closed_form():
    rng = np.random.default_rng(4)
    T, k, E = 50, 3, 7
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[:, :] = np.where(ids == 6, 5, ids)  # expert 6 never routed
    ids[0] = [0, 1, 2]
    w = rng.uniform(0.1, 1.0, (T, k))
    norms = rng.uniform(0.5, 3.0, T * k)
    got = moe.reap_saliency(norms, w, ids, E)
    for e in range(E):
        num, cnt = 0.0, 0
        for p in range(T * k):
            if ids.reshape(-1)[p] == e:
                num += w.reshape(-1)[p] * norms[p]
                cnt += 1
        want = num / cnt if cnt else 0.0
        assert abs(got[e] - want) <= 1e-12 * max(1.0, abs(want))
    assert got[6] == 0.0
    # closed form: constant norm n per pair -> S_e = n * mean routed weight
    got2 = moe.reap_saliency(np.full(T * k, 2.0), w, ids, E)
    for e in range(6):
        m = w.reshape(-1)[ids.reshape(-1) == e]
        if m.size:
            assert abs(got2[e] - 2.0 * m.mean()) < 1e-12


def test_layer_saliency_uses_unweighted_f_and_rsf_weights():
    T, H, I, E, k = 6, 32, 16, 4, 2
    x, wr, bias, experts, gs_x, gs_h = _rand_layer(13, T, H, I, E)
    out = moe.moe_layer(x, wr, bias, k, 2.5, gs_x, experts, gs_h, with_pairs=True)
    norms = np.linalg.norm(out["pair_f"], axis=1)
    assert np.allclose(out["pair_norm"], norms, rtol=1e-14)
    w = out["weights64"].reshape(-1)
    flat = out["ids"].reshape(-1)
    for e in range(E):
        sel = flat == e
        want = (w[sel] * norms[sel]).mean() if sel.any() else 0.0
        assert abs(out["saliency"][e] - want) <= 1e-12 * max(1.0, want)
    # combine: y_t = sum_j w_tj f_p
    y = np.zeros_like(out["y"])
    for p in range(T * k):
        y[p // k] += w[p] * out["pair_f"][p]
    assert np.allclose(out["y"], y, rtol=0, atol=1e-12 * np.abs(y).max())


def test_token_subset_matches_full_layer():
    T, H, I, E, k = 10, 32, 16, 4, 2
    x, wr, bias, experts, gs_x, gs_h = _rand_layer(17, T, H, I, E)
    full = moe.moe_layer(x, wr, bias, k, 2.5, gs_x, experts, gs_h)
    sub = moe.moe_layer(x, wr, bias, k, 2.5, gs_x, experts, gs_h, tokens=[7, 2])
    assert np.array_equal(sub["ids"], full["ids"][[7, 2]])
    assert np.allclose(sub["y"], full["y"][[7, 2]], rtol=0, atol=1e-13 * np.abs(full["y"]).max())


def test_calibration_definition():
    T, H, I, E = 2, 32, 16, 3
    x, wr, bias, experts, _, _ = _rand_layer(23, T, H, I, E)
    rng = np.random.default_rng(99)
    xc = _bf16(rng.standard_normal((16, H)))
    gs_x, gs_h = moe.calibrate(xc, experts, E)
    xf = gen.bf16_bits_to_f32(xc)
    assert gs_x == np.float32(np.float32(2688.0) / np.float32(np.max(np.abs(xf))))
    codes, scales = nvfp4.quantize(xf, gs_x)
    xhat = nvfp4.dequantize(codes, scales, gs_x)
    for e in range(E):
        wg, wu, _ = experts[e].dequantized()
        g, u = xhat @ wg.T, xhat @ wu.T
        h = (g / (1 + np.exp(-g)) * u).astype(np.float32)
        assert gs_h[e] == np.float32(np.float32(2688.0) / np.max(np.abs(h)))
    # the calibration amax maps to the top code at the top scale
    assert moe.calibrate(xc, experts, E, threads=3)[1].tolist() == gs_h.tolist()


def test_expert_pairs_output_equals_layer_pairs_and_loops():
    """expert_pairs_output (the per-expert reference of the full-size checks) gives the
    layer's own unweighted f for the same pairs, and a pure-Python loop on one expert:
    a dropped NVFP4 quantization of x or of h, the wrong gs_h or a transposed weight
    fails here."""
    T, H, I, E, k = 7, 32, 16, 4, 2
    x, wr, bias, experts, gs_x, gs_h = _rand_layer(31, T, H, I, E)
    out = moe.moe_layer(x, wr, bias, k, 2.5, gs_x, experts, gs_h, with_pairs=True)
    flat = out["ids"].reshape(-1)
    checked = 0
    for e in range(E):
        pairs = np.nonzero(flat == e)[0]
        if len(pairs) == 0:
            continue
        f = moe.expert_pairs_output(x[pairs // k], gs_x, experts[e], gs_h[e])
        want = out["pair_f"][pairs]
        assert np.max(np.abs(f - want)) <= 1e-13 * np.max(np.abs(want))
        checked += 1
    assert checked >= 2
    # loops for expert 1 on three token rows, from the pinned quantizer and math.fsum
    e, rows = 1, [0, 3, 6]
    W = experts[e]
    wg = nvfp4.dequantize_packed(W.gate_codes, W.gate_scales, W.gate_gs)
    wu = nvfp4.dequantize_packed(W.up_codes, W.up_scales, W.up_gs)
    wd = nvfp4.dequantize_packed(W.down_codes, W.down_scales, W.down_gs)
    got = moe.expert_pairs_output(x[rows], gs_x, W, gs_h[e])
    for n, t in enumerate(rows):
        xf = gen.bf16_bits_to_f32(x[t:t + 1])
        xc, xs = nvfp4.quantize(xf, gs_x)
        xhat = nvfp4.dequantize(xc, xs, gs_x)[0]
        h = []
        for i in range(I):
            g = math.fsum(xhat[c] * wg[i, c] for c in range(H))
            u = math.fsum(xhat[c] * wu[i, c] for c in range(H))
            h.append(float(np.float32(g / (1.0 + math.exp(-g)) * u)))
        hc, hs = nvfp4.quantize(np.array([h], np.float32), gs_h[e])
        hhat = nvfp4.dequantize(hc, hs, gs_h[e])[0]
        for o in range(H):
            f = math.fsum(hhat[i] * wd[o, i] for i in range(I))
            assert abs(got[n, o] - f) <= 1e-12 * max(1.0, abs(f))


def test_layer_threads_do_not_change_results():
    T, H, I, E, k = 9, 32, 16, 5, 2
    x, wr, bias, experts, gs_x, gs_h = _rand_layer(37, T, H, I, E)
    a = moe.moe_layer(x, wr, bias, k, 2.5, gs_x, experts, gs_h, with_pairs=True)
    b = moe.moe_layer(x, wr, bias, k, 2.5, gs_x, experts, gs_h, with_pairs=True, threads=4)
    for key in ("ids", "y", "saliency", "pair_norm", "pair_f"):
        assert np.array_equal(a[key], b[key]), key
