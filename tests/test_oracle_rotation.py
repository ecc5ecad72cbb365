"""Pins of the Hadamard rotation oracle (oracle/rotation.py): the Sylvester
construction, butterfly brute force, orthogonality, exact invariance of the
products it is applied to, and the unquantized reference layer."""

import math

import numpy as np
import pytest

from oracle import nvfp4 as onv
from oracle import rotation as orot
from oracle import routing as oroute
from workloads import WEIGHT_SETS, gen


def bf(a):
    return gen.f32_to_bf16_bits(np.asarray(a, np.float32))


def test_sylvester_small_and_orthogonal():
    assert np.array_equal(orot.sylvester(1), [[1]])
    assert np.array_equal(orot.sylvester(4), [[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]])
    for b in (2, 8, 64, 256):
        h = orot.sylvester(b)
        assert set(np.unique(h)) == {-1.0, 1.0}
        assert np.array_equal(h @ h.T, b * np.eye(b))
    with pytest.raises(ValueError):
        orot.sylvester(12)


def _fwht(v):
    """In-place butterflies (the fast transform), pure Python, unnormalized."""
    v = list(v)
    n, h = len(v), 1
    while h < n:
        for i in range(0, n, 2 * h):
            for j in range(i, i + h):
                v[j], v[j + h] = v[j] + v[j + h], v[j] - v[j + h]
        h *= 2
    return v


def test_rotation_equals_butterflies():
    rng = np.random.default_rng(0)
    n = 64
    for b in (2, 8, 32, 64):
        v = rng.standard_normal(n)
        s = rng.choice([-1.0, 1.0], n)
        got = orot.rotate_rows(v[None], s, b)[0]
        want = []
        for blk in range(n // b):
            want += [x / math.sqrt(b) for x in _fwht(list(v[blk * b:(blk + 1) * b] * s[blk * b:(blk + 1) * b]))]
        assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_one_hot_and_norm():
    n, b = 32, 16
    s = np.where(np.arange(n) % 3 == 0, -1.0, 1.0)
    e = np.zeros(n)
    e[19] = 2.0
    r = orot.rotate_rows(e[None], s, b)[0]
    assert np.all(r[:16] == 0) and np.allclose(np.abs(r[16:]), 2.0 / 4.0)  # spread over its block, +-2/sqrt(16)
    rng = np.random.default_rng(1)
    v = rng.standard_normal((5, 2048))
    s = rng.choice([-1.0, 1.0], 2048)
    for b in (16, 128, 2048):
        assert np.allclose(np.linalg.norm(orot.rotate_rows(v, s, b), axis=1), np.linalg.norm(v, axis=1), rtol=1e-12)


def test_products_are_invariant():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 256))
    w = rng.standard_normal((9, 256))
    s = rng.choice([-1.0, 1.0], 256)
    for b in (4, 64, 256):
        assert np.allclose(orot.rotate_rows(x, s, b) @ orot.rotate_rows(w, s, b).T, x @ w.T, rtol=1e-11, atol=1e-11)


def test_rotate_bf16_is_the_rounded_rotation():
    rng = np.random.default_rng(3)
    x = bf(rng.standard_normal((4, 128)))
    s = rng.choice([-1.0, 1.0], 128)
    got = gen.bf16_bits_to_f32(orot.rotate_bf16(x, s, 128)).astype(np.float64)
    exact = orot.rotate_rows(gen.bf16_bits_to_f32(x), s, 128)
    assert np.all(np.abs(got - exact) <= np.abs(exact) * 2.0 ** -8)


def test_reference_layer_brute_force():
    rng = np.random.default_rng(4)
    T, H, I, E, k, rsf = 3, 8, 4, 3, 2, 2.5
    x = bf(rng.standard_normal((T, H)))
    wr = bf(rng.standard_normal((E, H)))
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    ex = [tuple(bf(rng.standard_normal(sh) * 0.5) for sh in ((I, H), (I, H), (H, I))) for _ in range(E)]
    out = orot.moe_layer_reference(x, wr, bias, k, rsf, lambda e: ex[e])
    ids, _, w64, _ = oroute.route(x, wr, bias, k, rsf)
    f = lambda b: float(gen.bf16_bits_to_f32(np.array([b], np.uint16))[0])  # noqa: E731
    for t in range(T):
        for n in range(H):
            acc = 0.0
            for j in range(k):
                g_, u_, d_ = ex[ids[t, j]]
                hsum = 0.0
                for c in range(I):
                    gg = sum(f(x[t, m]) * f(g_[c, m]) for m in range(H))
                    uu = sum(f(x[t, m]) * f(u_[c, m]) for m in range(H))
                    hsum += gg / (1 + math.exp(-gg)) * uu * f(d_[n, c])
                acc += w64[t, j] * hsum
            assert math.isclose(out["y"][t, n], acc, rel_tol=1e-10, abs_tol=1e-12)


def _rel(res, w, mask=None):
    w = gen.bf16_bits_to_f32(w).astype(np.float64)
    if mask is not None:
        res, w = res[mask], w[mask]
    return float(np.linalg.norm(res) / np.linalg.norm(w))


def test_quantization_residual():
    # a weight exactly representable in NVFP4 (codes x power-of-two block scales) has no residual unrotated
    rng = np.random.default_rng(5)
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    w = rng.choice(vals, (16, 64)) * rng.choice([-1, 1], (16, 64))
    w[:, ::16] = 6.0  # every block reaches the E2M1 maximum
    assert not np.any(orot.quantization_residual(bf(w / 8)))
    # rotating back is exact up to the BF16 rounding of the rotated values when nothing is lost to NVFP4:
    # a rotated one-hot row is +-1/sqrt(b) in one block, representable, so the residual is 0
    e = np.zeros((1, 64))
    e[0, 5] = 1.0
    s = np.ones(64)
    assert np.allclose(orot.quantization_residual(bf(e), s, 16), 0.0, atol=1e-15)


def _kurtosis(a):
    a = np.asarray(a, np.float64).reshape(-1)
    a = a - a.mean()
    return float(np.mean(a ** 4) / np.mean(a ** 2) ** 2)


def test_rotation_gaussianizes_the_outlier_recipe():
    """A 2048-wide rotation sums 2048 signed entries per output: the heavy-tail recipe's rows become
    Gaussian (kurtosis 3), which is what removes the outliers NVFP4's block scales see."""
    ws = WEIGHT_SETS["e128_outlier"]
    g, _, _ = gen.expert_bf16(ws, 0)
    w = g[:32]
    s = gen.rotation_signs(ws.H)
    before = _kurtosis(gen.bf16_bits_to_f32(w))
    after = _kurtosis(gen.bf16_bits_to_f32(orot.rotate_bf16(w, s, 2048)))
    assert before > 20 and abs(after - 3.0) < 0.3, (before, after)


def test_residual_norm_is_the_rotated_one():
    """||Q R^T - W|| = ||Q - W R|| (R orthogonal): the residual mapped back keeps its norm."""
    rng = np.random.default_rng(7)
    w = bf(rng.standard_normal((8, 512)) * 0.02)
    s = rng.choice([-1.0, 1.0], 512)
    for b in (16, 128, 512):
        back = orot.quantization_residual(w, s, b)
        wr = gen.bf16_bits_to_f32(orot.rotate_bf16(w, s, b))
        q = onv.dequantize_packed(*onv.quantize_weight(wr))
        exact_rot = orot.rotate_rows(gen.bf16_bits_to_f32(w), s, b)
        assert np.isclose(np.linalg.norm(back), np.linalg.norm(q - exact_rot), rtol=1e-10)


def test_rotation_keeps_gaussian_error():
    ws = WEIGHT_SETS["e128_outlier"]
    s = gen.rotation_signs(ws.H)
    w_gauss = bf(np.random.default_rng(6).standard_normal((32, ws.H)) * 0.02)
    ratio = _rel(orot.quantization_residual(w_gauss, s, 2048), w_gauss) / _rel(orot.quantization_residual(w_gauss),
                                                                               w_gauss)
    assert 0.9 < ratio < 1.1, ratio
