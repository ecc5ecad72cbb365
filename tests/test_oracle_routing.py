"""Pins for the oracle's routing and permutation (CPU): a hand-derived example
with closed-form weights, the rsf sum invariant, subset brute force, bias
shift invariance, ties, and the stable-sort definition of the permutation."""

import itertools
import math

import numpy as np
import pytest

from oracle import routing
from workloads import by_name, gen


def _bf16(vals):
    return gen.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_hand_example_bias_selects_weights_renormalize_sigmoid():
    """x = [1, 0]; router rows give logits [0, 1, -1, 0.5]; bias [0.3, 0, 0, 0].

    scores = sigmoid + bias = [0.8, 0.731, 0.269, 0.622] -> top-2 = experts 0, 1.
    Weights renormalize the bias-free sigmoid: with s0 = 1/2, s1 = e/(1+e),
    w0 = rsf (1+e)/(1+3e) and w1 = rsf 2e/(1+3e)."""
    x = _bf16([[1.0, 0.0]])
    w = _bf16([[0.0, 0.0], [1.0, 0.0], [-1.0, 0.0], [0.5, 0.0]])
    bias = np.array([0.3, 0.0, 0.0, 0.0], np.float32)
    rsf = 2.5
    ids, w32, w64, gap = routing.route(x, w, bias, 2, rsf)
    assert ids.tolist() == [[0, 1]]
    e = math.e
    assert abs(w64[0, 0] - rsf * (1 + e) / (1 + 3 * e)) < 1e-15
    assert abs(w64[0, 1] - rsf * 2 * e / (1 + 3 * e)) < 1e-15
    # without the bias the choice would be experts 1 and 3
    ids_nb, *_ = routing.route(x, w, np.zeros(4, np.float32), 2, rsf)
    assert ids_nb.tolist() == [[1, 3]]
    # margin to the first excluded expert (3): 0.731 - 0.622
    assert abs(gap[0] - (e / (1 + e) - 1 / (1 + math.exp(-0.5)))) < 1e-15


def test_logits_are_exact_bf16_products_in_float64():
    rng = np.random.default_rng(1)
    x = _bf16(rng.standard_normal((3, 64)))
    w = _bf16(rng.standard_normal((5, 64)) * 0.02)
    lg = routing.router_logits(x, w)
    xf, wf = gen.bf16_bits_to_f32(x), gen.bf16_bits_to_f32(w)
    for t in range(3):
        for e in range(5):
            exact = math.fsum(float(a) * float(b) for a, b in zip(xf[t], wf[e]))
            assert abs(lg[t, e] - exact) <= 1e-15 * max(1.0, abs(exact))


@pytest.fixture(scope="module")
def tiny():
    cfg = by_name("tiny")
    x = gen.tokens(cfg)
    wr = gen.router_weight(cfg.weights)
    b = gen.router_bias(cfg)
    return cfg, x, wr, b


def test_weights_sum_to_rsf(tiny):
    cfg, x, wr, b = tiny
    ids, w32, w64, gap = routing.route(x, wr, b, cfg.k, cfg.rsf)
    assert np.all(np.abs(w64.sum(1) - cfg.rsf) <= 1e-12 * cfg.rsf)
    assert np.all(np.abs(w32.astype(np.float64).sum(1) - cfg.rsf) <= 1e-6 * cfg.rsf)
    assert np.all(w64 > 0)


def test_topk_is_best_subset_by_brute_force(tiny):
    """The selected set maximizes the summed score over all C(E,k) subsets."""
    cfg, x, wr, b = tiny
    lg = routing.router_logits(x, wr)
    ids, *_ = routing.select_topk(lg, b, cfg.k, cfg.rsf)
    score = 1 / (1 + np.exp(-lg)) + b.astype(np.float64)
    for t in range(x.shape[0]):
        best = max(itertools.combinations(range(cfg.E), cfg.k), key=lambda c: sum(score[t, list(c)]))
        assert sorted(ids[t].tolist()) == sorted(best)
        # slots ordered by descending score
        assert np.all(np.diff(score[t, ids[t]]) <= 0)


def test_bias_shift_invariance(tiny):
    cfg, x, wr, b = tiny
    a = routing.route(x, wr, b, cfg.k, cfg.rsf)
    c = routing.route(x, wr, (b + np.float32(0.25)).astype(np.float32), cfg.k, cfg.rsf)
    assert np.array_equal(a[0], c[0])
    assert np.array_equal(a[1], c[1])


def test_ties_go_to_lower_index():
    lg = np.zeros((2, 5))
    lg[1, 3] = 1.0
    ids, w32, _, gap = routing.select_topk(lg, np.zeros(5, np.float32), 3, 1.0)
    assert ids[0].tolist() == [0, 1, 2]
    assert ids[1].tolist() == [3, 0, 1]
    assert gap[0] == 0.0  # a true tie at the boundary is reported
    assert np.allclose(w32[0], 1 / 3)


def test_k_equals_e_selects_everything():
    lg = np.random.default_rng(0).standard_normal((4, 6))
    ids, w32, w64, gap = routing.select_topk(lg, np.zeros(6, np.float32), 6, 2.5)
    assert all(sorted(r) == list(range(6)) for r in ids.tolist())
    assert np.all(np.isinf(gap))


def test_permutation_is_python_stable_sort(tiny):
    cfg, x, wr, b = tiny
    ids, *_ = routing.route(x, wr, b, cfg.k, cfg.rsf)
    counts, offsets, perm = routing.permute(ids, cfg.E)
    flat = ids.reshape(-1).tolist()
    want = sorted(range(len(flat)), key=lambda p: flat[p])  # Python's sort is stable
    assert perm.tolist() == want
    assert counts.sum() == len(flat)
    assert offsets[0] == 0 and offsets[-1] == len(flat)
    assert np.all(np.diff(offsets) == counts)
    for e in range(cfg.E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert all(flat[p] == e for p in seg)
        assert np.all(np.diff(seg) > 0)


def test_permutation_handles_empty_experts_and_no_tokens():
    counts, offsets, perm = routing.permute(np.zeros((0, 2), np.int32), 4)
    assert counts.tolist() == [0, 0, 0, 0] and offsets.tolist() == [0] * 5 and perm.size == 0
    counts, offsets, perm = routing.permute(np.array([[3, 3], [3, 0]], np.int32), 5)
    assert counts.tolist() == [1, 0, 0, 3, 0]
    assert offsets.tolist() == [0, 1, 1, 1, 4, 4]
    assert perm.tolist() == [3, 0, 1, 2]
