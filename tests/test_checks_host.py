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
