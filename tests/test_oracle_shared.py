"""Pins of the shared-expert oracle (oracle/shared.py): closed forms, brute force and invariants."""

import math

import numpy as np

from oracle import shared as osh
from workloads import gen


def bf(a):
    return gen.f32_to_bf16_bits(np.asarray(a, np.float32))


def test_round_bf16_grid_and_ties():
    r = osh.round_bf16
    assert r(np.array([1.0]))[0] == 1.0
    # spacing next to 1 is 2^-7: midpoints go to the even significand
    assert r(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert r(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert r(np.array([1.0 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1.0 + 2.0 ** -7
    assert r(np.array([-3.0 - 2.0 ** -7]))[0] == -3.0  # 3 = 1.1b x 2^1, spacing 2^-6: tie to even
    assert r(np.array([0.0, -0.0]))[1] == 0.0 and np.signbit(r(np.array([-0.0]))[0])
    assert r(np.array([2.0 ** -133]))[0] == 2.0 ** -133  # smallest BF16 subnormal
    assert r(np.array([3 * 2.0 ** -135]))[0] == 2.0 ** -133  # 0.75 step rounds up
    assert np.isinf(r(np.array([3.4e38]))[0])


def test_round_bf16_against_the_f32_bit_route():
    """For float32 inputs, the result equals the bit-level RNE of the input generators."""
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(20000) * np.exp2(rng.integers(-60, 60, 20000))).astype(np.float32)
    want = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(a)).astype(np.float64)
    assert np.array_equal(osh.round_bf16(a.astype(np.float64)), want)


def test_round_bf16_is_nearest():
    """Brute force: the result is a BF16 value and no BF16 neighbour is closer."""
    rng = np.random.default_rng(1)
    a = rng.standard_normal(5000) * np.exp2(rng.uniform(-20, 20, 5000))
    r = osh.round_bf16(a)
    bits = gen.f32_to_bf16_bits(r.astype(np.float32))
    assert np.array_equal(gen.bf16_bits_to_f32(bits).astype(np.float64), r)  # exactly a BF16 value
    for d in (-1, 1):  # the neighbouring BF16 values, by bit pattern
        nb = gen.bf16_bits_to_f32((bits.astype(np.int32) + d).astype(np.uint16)).astype(np.float64)
        assert np.all(np.abs(a - r) <= np.abs(a - nb))


def test_one_hot_closed_form():
    """x = a e_i, W_gate[c] = b e_i, W_up[c] = d e_i, W_down = identity: s = bf16(silu(ab) * ad)."""
    H = I = 16
    a, b, d = 1.5, -0.75, 2.5
    x = np.zeros((1, H), np.float32)
    x[0, 3] = a
    wg = np.zeros((I, H), np.float32)
    wu = np.zeros((I, H), np.float32)
    wg[:, 3] = b * np.arange(1, I + 1) / 8  # column c gets b * (c+1)/8 (exact in BF16)
    wu[:, 3] = d
    wd = np.eye(H, I, dtype=np.float32)
    s, h = osh.shared_expert(bf(x), bf(wg), bf(wu), bf(wd))
    for c in range(I):
        z = a * b * (c + 1) / 8
        want = z / (1.0 + math.exp(-z)) * (a * d)
        assert abs(h[0, c] - want) <= abs(want) * 2.0 ** -8
        assert s[0, c] == h[0, c]


def test_brute_force_tiny():
    rng = np.random.default_rng(2)
    T, H, I = 3, 8, 4
    x = bf(rng.standard_normal((T, H)))
    wg, wu = bf(rng.standard_normal((I, H))), bf(rng.standard_normal((I, H)))
    wd = bf(rng.standard_normal((H, I)))
    s, h = osh.shared_expert(x, wg, wu, wd)
    f = lambda b: float(gen.bf16_bits_to_f32(np.array([b], np.uint16))[0])  # noqa: E731
    for t in range(T):
        hh = []
        for c in range(I):
            g = sum(f(x[t, j]) * f(wg[c, j]) for j in range(H))
            u = sum(f(x[t, j]) * f(wu[c, j]) for j in range(H))
            v = g / (1.0 + math.exp(-g)) * u
            assert abs(h[t, c] - v) <= abs(v) * 2.0 ** -8 + 1e-300
            hh.append(h[t, c])
        for n in range(H):
            assert math.isclose(s[t, n], sum(hh[c] * f(wd[n, c]) for c in range(I)), rel_tol=1e-12, abs_tol=1e-12)


def test_invariants():
    rng = np.random.default_rng(3)
    T, H, I = 5, 32, 16
    x = bf(rng.standard_normal((T, H)))
    wg, wu = bf(rng.standard_normal((I, H)) * 0.1), bf(rng.standard_normal((I, H)) * 0.1)
    wd = bf(rng.standard_normal((H, I)) * 0.1)
    s, h = osh.shared_expert(x, wg, wu, wd)
    neg = lambda w: bf(-gen.bf16_bits_to_f32(w))  # noqa: E731  exact negation
    s2, h2 = osh.shared_expert(x, wg, neg(wu), wd)
    assert np.array_equal(h2, -h) and np.array_equal(s2, -s)  # u -> -u flips the sign exactly
    s3, _ = osh.shared_expert(x, wg, wu, bf(2 * gen.bf16_bits_to_f32(wd)))
    assert np.array_equal(s3, 2 * s)  # power-of-two scaling of W_down is exact
    s4, h4 = osh.shared_expert(x, wg, bf(np.zeros((I, H))), wd)
    assert not np.any(h4) and not np.any(s4)
    y = rng.standard_normal((T, H))
    assert np.array_equal(osh.block_output(y, s4), y)  # no shared contribution: the routed output
    # h is the input of a BF16 Linear: every value is a BF16 value
    assert np.array_equal(gen.bf16_bits_to_f32(bf(h)).astype(np.float64), h)
