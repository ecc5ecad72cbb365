"""Host-only pins for the parity checkers the GPU tests rely on (no GPU needed).

check_routing must accept any valid top-k for tokens whose oracle margin is
below NEAR_TIE (an exact tie included) and reject an invalid one: a choice
outside the top-k, a wrong slot order, a repeated id, or weights that are not
the renormalized sigmoid over the chosen set.
"""

import numpy as np
import pytest

from gpu_cases import NEAR_TIE, check_routing
from oracle import routing as oroute
from workloads import gen


def _tied_case():
    rng = np.random.default_rng(3)
    T, H, E, k = 6, 32, 8, 3
    wr = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    wr[5] = wr[2]  # experts 2 and 5 tie exactly on every token
    bias = np.zeros(E, np.float32)
    bias[2] = bias[5] = 1.0  # ... and lead every token
    xb = gen.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wrb = gen.f32_to_bf16_bits(wr)
    ids, w32, w64, gap = oroute.route(xb, wrb, bias, k, 2.5)
    return xb, wrb, bias, E, k, ids, w32, {"ids": ids, "weights64": w64, "gap": gap}


def test_exact_tie_swapped_slots_are_valid():
    xb, wrb, bias, E, k, ids, w32, ref = _tied_case()
    assert np.all(ids[:, :2] == [2, 5])
    # put token 0's margin below NEAR_TIE so it takes the validation path, then swap its tied slots
    ref = dict(ref, gap=ref["gap"].copy())
    ref["gap"][0] = 0.0
    g_ids, g_w = ids.copy(), w32.copy()
    g_ids[0, [0, 1]] = g_ids[0, [1, 0]]
    g_w[0, [0, 1]] = g_w[0, [1, 0]]
    assert check_routing(g_ids, g_w, ref, 2.5, E, xb, wrb, bias) == 1


@pytest.mark.parametrize("mutation", ["outside_topk", "repeated_id", "slot_order", "weights", "no_inputs",
                                      "clear_token_differs"])
def test_invalid_choices_are_rejected(mutation):
    xb, wrb, bias, E, k, ids, w32, ref = _tied_case()
    ref = dict(ref, gap=ref["gap"].copy())
    ref["gap"][0] = 0.0
    g_ids, g_w = ids.copy(), w32.copy()
    args = (xb, wrb, bias)
    if mutation == "outside_topk":
        s = oroute.sigmoid(oroute.router_logits(xb[:1], wrb))[0] + bias
        worst = int(np.argmin(s))
        g_ids[0, k - 1] = worst
    elif mutation == "repeated_id":
        g_ids[0, 2] = g_ids[0, 0]
    elif mutation == "slot_order":
        g_ids[0, [0, 2]] = g_ids[0, [2, 0]]
    elif mutation == "weights":
        g_w[0, 0] *= 1.001
    elif mutation == "no_inputs":
        args = ()
    elif mutation == "clear_token_differs":
        g_ids[1, [1, 2]] = g_ids[1, [2, 1]]
        ref["gap"][1] = 1.0
    with pytest.raises(AssertionError):
        check_routing(g_ids, g_w, ref, 2.5, E, *args)


def test_expected_pair_scale_rule():
    """The row-scale rule the GPU pair rows are checked against: 2^E with B * 2^-E in [2^14, 2^15) for every bound
    in FP32's normal range not clamped, so the largest value any FP4 operands allow stays below FP16's 65504; the
    exponent clamps at -126 and 113; the scale is a power of two."""
    from gpu_cases import expected_pair_scale

    rng = np.random.default_rng(5)
    n = 20000
    w = rng.uniform(0.0, 3.0, n).astype(np.float32)
    w[:5] = [0.0, 1e-30, 2.5, np.float32(2.0 ** -126), 1.0]
    ids = rng.integers(0, 4, n)
    h_gs = np.float32(10.0) ** rng.uniform(-3, 12, 4).astype(np.float32)
    w2_gs = np.float32(10.0) ** rng.uniform(-3, 6, 4).astype(np.float32)
    I = 2048
    sc = expected_pair_scale(w, ids, I, h_gs, w2_gs)
    m, e = np.frexp(sc)
    assert np.all(m == 0.5)  # powers of two
    E = e.astype(np.int64) - 1
    assert E.min() >= -126 and E.max() <= 113
    bound = (w.astype(np.float64) * I * 2688.0 ** 2) / (h_gs[ids].astype(np.float64) * w2_gs[ids].astype(np.float64))
    scaled = bound * np.ldexp(1.0, -E)
    free = (E > -126) & (E < 113)
    assert np.all(scaled[free] < 2.0 ** 15 * (1 + 1e-6)) and np.all(scaled[free] >= 2.0 ** 14 * (1 - 1e-6))
    assert np.all(scaled < 2.0 ** 15 * (1 + 1e-6))  # clamped at the bottom: smaller still
    assert np.all(E[w == 0] == -126)
    # an FP16 value below 2^15 times the scale is exact in FP32, as the combine relies on
    big = np.float16(32752.0).astype(np.float32) * sc  # largest FP16 below 2^15
    assert np.all(np.isfinite(big))
