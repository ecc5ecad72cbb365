"""Host check of the selection order the routing kernel ranks by (no GPU needed).

The kernel maps each FP64 score to a 64-bit integer key -- NaN below every
number, -0 equal to +0, negatives by flipping their magnitude bits -- and ranks
experts by (key descending, index ascending).  This restates that rule in
Python and checks that it yields the oracle's top-k (a stable descending sort
of the scores, NaN last) on rows with NaN, +-inf, +-0, subnormals and exact
ties, and that every rank 0..E-1 is taken once, so every top-k slot is written.
"""

import numpy as np
import pytest

from oracle import routing as oroute

INT64_MIN = -(1 << 63)


def score_key(v: float) -> int:
    if v != v:
        return INT64_MIN
    b = int(np.array([v], np.float64).view(np.int64)[0])
    if b == INT64_MIN:  # -0
        b = 0
    return b ^ 0x7FFFFFFFFFFFFFFF if b < 0 else b


def kernel_ranks(scores: np.ndarray) -> list[int]:
    keys = [score_key(float(v)) for v in scores]
    E = len(keys)
    return [sum(1 for f in range(E) if keys[f] > keys[e] or (keys[f] == keys[e] and f < e)) for e in range(E)]


def kernel_topk(scores: np.ndarray, k: int) -> list[int]:
    ranks = kernel_ranks(scores)
    slots = [-1] * k
    for e, r in enumerate(ranks):
        if r < k:
            slots[r] = e
    return slots


def _rows():
    rng = np.random.default_rng(11)
    nan, inf = np.nan, np.inf
    rows = [
        np.full(8, nan),
        np.array([0.3, nan, 0.7, -0.0, 0.0, nan, -inf, inf]),
        np.array([-0.0, 0.0, -0.0, 0.0, 5e-324, -5e-324, 1.0, -1.0]),
        np.array([0.5, 0.5, 0.5, nan, 0.5, -inf, -inf, 0.2]),
        np.array([-inf, -inf, nan, -inf, -1e308, -2.0, nan, -inf]),
        np.array([1.5, 1.5 + 2e-16, 1.5 - 2e-16, 1.5, 1.0, 2.0, 2.0, nan]),
    ]
    for _ in range(40):
        r = rng.choice([0.1, 0.2, 0.3, -0.3, 0.0, -0.0, np.nan, np.inf, -np.inf, 1e-310, -1e-310], size=13)
        rows.append(r.astype(np.float64))
    return rows


def _bias_rows():
    """float32 biases whose score 0.5 + bias (zero logits) is exact in float64."""
    rng = np.random.default_rng(12)
    f = np.float32
    nan, inf = f(np.nan), f(np.inf)
    rows = [
        np.full(8, nan, f),
        np.array([0.25, nan, 0.75, -0.5, 0.0, nan, -inf, inf], f),
        np.array([0.125, 0.125, 0.125, nan, 0.125, -inf, -inf, -0.375], f),
        np.array([-inf, -inf, nan, -inf, -1e30, -2.0, nan, -inf], f),
        np.array([1.5, 1.5, 1.25, 1.5, 1.0, 2.0, 2.0, nan], f),
    ]
    vals = np.array([0.1, 0.2, 0.3, -0.3, 0.0, -0.5, np.nan, np.inf, -np.inf, 2.0 ** -20], f)
    for _ in range(40):
        rows.append(rng.choice(vals, size=13))
    return rows


@pytest.mark.parametrize("i", range(45))
def test_key_order_matches_oracle_selection(i):
    bias = _bias_rows()[i]
    E = len(bias)
    sc = 0.5 + bias.astype(np.float64)  # the oracle's score at logit 0: sigmoid(0) + bias
    ranks = kernel_ranks(sc)
    assert sorted(ranks) == list(range(E))  # a permutation: every slot written exactly once
    for k in sorted({1, 2, E // 2, E}):
        ids, *_ = oroute.select_topk(np.zeros((1, E)), bias, k, 1.0)
        assert ids[0].tolist() == kernel_topk(sc, k)


@pytest.mark.parametrize("i", range(46))
def test_key_order_is_stable_descending_nan_last(i):
    """Signed zeros and subnormals too: the order of a stable descending sort with NaN last."""
    sc = _rows()[i]
    E = len(sc)
    assert sorted(kernel_ranks(sc)) == list(range(E))
    assert kernel_topk(sc, E) == np.argsort(-sc, kind="stable").tolist()
