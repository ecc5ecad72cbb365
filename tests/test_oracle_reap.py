"""Pins of the REAP pruning oracle (oracle/reap.py) against properties the pages and its definition fix."""

import itertools

import numpy as np
import pytest

from oracle import moe as omoe
from oracle import reap as oreap
from oracle import routing as oroute


def test_keep_ids_brute_force_small():
    """Exhaustive check on tiny inputs with many ties: the kept set maximizes saliency, ties to lower index."""
    rng = np.random.default_rng(0)
    for _ in range(200):
        E = int(rng.integers(1, 7))
        s = rng.integers(0, 3, E).astype(np.float32)  # few distinct values: many ties
        for n in range(1, E + 1):
            got = oreap.keep_ids(s, n)
            # brute force: among all n-subsets, maximize (sum of saliencies as a sorted tuple), then prefer
            # lexicographically smallest index set -- equivalent to keeping the n best under (s desc, index asc)
            best = None
            for sub in itertools.combinations(range(E), n):
                key = (sorted((-float(s[e]) for e in sub)), sub)
                if best is None or key < best[0]:
                    best = (key, sub)
            assert tuple(got.tolist()) == best[1], (s, n)


def test_keep_ids_invariants():
    rng = np.random.default_rng(1)
    s = rng.random(128).astype(np.float32)
    s[rng.choice(128, 10, replace=False)] = 0.0  # never-routed experts
    keep = oreap.keep_ids(s, 80)
    assert keep.shape == (80,) and np.all(np.diff(keep) > 0)  # ascending, distinct
    dropped = np.setdiff1d(np.arange(128), keep)
    assert dropped.shape == (48,)  # the pages' 128 -> 80: 48 removed
    assert s[keep].min() >= s[dropped].max()
    assert np.all(np.isin(np.nonzero(s == 0.0)[0], dropped))  # zero-saliency experts go first


def test_keep_ids_special_cases():
    assert oreap.keep_ids(np.zeros(5, np.float32), 3).tolist() == [0, 1, 2]  # all tied: lowest indices
    assert oreap.keep_ids(np.array([1, 2, 3], np.float32), 3).tolist() == [0, 1, 2]  # keep all
    assert oreap.keep_ids(np.array([3, 1, 2], np.float32), 1).tolist() == [0]
    with pytest.raises(ValueError):
        oreap.keep_ids(np.ones(4, np.float32), 0)


def test_pruned_routing_is_routing_over_the_kept_experts():
    """Slicing the router then routing equals routing with the dropped experts' scores removed."""
    rng = np.random.default_rng(2)
    T, H, E, k = 40, 32, 12, 3
    bf = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)  # truncation: exact bf16
    x = bf(rng.standard_normal((T, H)))
    wr = bf(rng.standard_normal((E, H)) * 0.1)
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    keep = np.array([0, 2, 3, 5, 8, 9, 11], np.int32)
    wr_k, b_k = oreap.slice_router(wr, bias, keep)
    ids_k, w_k, _, _ = oroute.route(x, wr_k, b_k, k, 2.5)
    # reference: full logits, scores of dropped experts set to -inf, same selection rule
    logits = oroute.router_logits(x, wr)
    sc = 1.0 / (1.0 + np.exp(-logits)) + bias.astype(np.float64)
    sc[:, np.setdiff1d(np.arange(E), keep)] = -np.inf
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-sc[t, e], e))[:k]
        assert [int(keep[i]) for i in ids_k[t]] == order
    assert np.allclose(w_k.sum(axis=1), 2.5, rtol=1e-6)  # renormalized over the kept top-k


def test_slice_experts_order():
    ex = [f"e{i}" for i in range(6)]
    assert oreap.slice_experts(ex, np.array([1, 4, 5])) == ["e1", "e4", "e5"]
