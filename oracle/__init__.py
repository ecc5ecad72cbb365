"""CPU oracle for the routed-expert NVFP4 W4A4 MoE layer.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, obviously-correct
statement of what the layer computes.  It exists to check the HIP path and is
imported only by ``tests/``, by ``__graft_entry__.smoke()`` and by the
``cpu_baseline`` leg of ``bench.py``.  The product path (the C-ABI library and
its Python binding) never imports, calls or links anything in here, and this
package never imports the product path.  The two share no code; only the
seeded input generators in ``workloads/`` feed both.

Sources (page titles and sections; the pages state *what* is computed):

* "K-EXAONE-152B-A23B-REAP-80E-NVFP4" model card, section "Quantization
  Setup": NVFP4 W4A4, FP4 E2M1 weights, group size 16, FP8 E4M3 block
  scales, activations dynamically quantized with calibrated global scales,
  round-to-nearest PTQ, per-expert Linear granularity, router kept in BF16.
* "[NetsPresso AQ Deep Dive] How to Quantize the K-EXAONE-236B Model to 4-Bit
  (NVFP4)", section "The Standard NVFP4 Serving Spec": the double-scale
  structure (a global scale combined with a block scale).
* "K-EXAONE-152B-A23B-REAP-80E-BF16" model card, section "Pruning Setup":
  renormalized sigmoid routing with the e_score_correction_bias,
  routed_scaling_factor, and the REAP saliency mean(topk_weight * ||f_e(x)||_2)
  over routed tokens.
* Forum post "1x Spark GB10: 236B unpruned K-EXAONE-236B-A23B serving ...",
  sections "Caveats" and "Repos": top-8-of-128 sigmoid routing.

Modules:
  formats  -- E2M1 / E4M3 value tables and round-to-nearest-even encoders
  nvfp4    -- NVFP4 quantize / dequantize / global scale
  routing  -- router logits, sigmoid+bias top-k, renormalization, permutation
  moe      -- expert SwiGLU FFN, weighted combine, REAP saliency, calibration

Pinning status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` against closed forms, brute force, hand-derived
golden values or invariants.  What the pages leave open (the global-scale
convention, tie rules, whether the bias enters the weights) is a reading that
each function's docstring states; it is not an unpinned function.
"""

from . import formats, nvfp4, routing, moe  # noqa: F401
