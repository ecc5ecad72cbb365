"""REAP expert pruning step (oracle).

What the pages fix ("K-EXAONE-152B-A23B-REAP-80E-BF16" model card, the
introduction and section "Pruning Setup"):

* one-shot pruning removes the 48 routed experts of lowest REAP saliency from a
  128-expert layer, keeping 80;
* the router's gate weight and its e_score_correction_bias are sliced to the
  retained experts, and the renormalized sigmoid routing is kept unchanged
  (the top-k is now taken among the retained experts);
* the saliency is the one of ``oracle.moe.reap_saliency``.

Readings (pages silent):

* experts are ranked by (saliency descending, expert index ascending): among
  equal saliencies the lower index is kept; an expert never routed to has
  saliency 0 and so goes first;
* the retained experts keep their original relative order (new index i is the
  i-th retained old index), so "sliced" is a row selection.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

from __future__ import annotations

import numpy as np


def keep_ids(saliency: np.ndarray, n_keep: int) -> np.ndarray:
    """The n_keep retained experts, ascending by index."""
    s = np.asarray(saliency)
    E = s.shape[0]
    if not 1 <= n_keep <= E:
        raise ValueError("need 1 <= n_keep <= E")
    # rank order: saliency descending, then index ascending
    order = sorted(range(E), key=lambda e: (-float(s[e]), e))
    return np.array(sorted(order[:n_keep]), dtype=np.int32)


def slice_router(w_router: np.ndarray, bias: np.ndarray, keep: np.ndarray):
    """Router weight rows and bias entries of the retained experts, in the new order."""
    keep = np.asarray(keep)
    return np.asarray(w_router)[keep], np.asarray(bias)[keep]


def slice_experts(experts, keep: np.ndarray) -> list:
    """Expert list of the pruned layer: new expert i is old expert keep[i]."""
    return [experts[int(e)] for e in np.asarray(keep)]
