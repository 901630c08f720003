"""Oracle: a plain, slow, float64 CPU statement of the attention-layer backward pass.

THIS PACKAGE IS TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it. The GPU library never calls it, shares no
code, header, table or constant with it, and must fail loudly (not fall back here)
when its compiled extension is missing.

What it follows (cited by page title and section, never by line):
  * "Hesper.Training.VerifiedBackward" API page: the forward and backward (VJP) specs
    for softmax, RoPE, RMSNorm, the scaled dot product and single-head attention, and
    the numerical-gradient verification helpers (sections "Softmax", "RoPE (Rotary
    Position Embedding)", "RMSNorm", "Scaled Dot-Product", "Attention (full
    single-head)", "Numerical Gradient Verification").
  * The Hesper pull-request commit log: linear backward as an outer-product dW plus a
    transposed dX, the per-layer reverse backward chain over saved activations, the
    residual passing the hidden gradient through unchanged, and the wrong-backward set
    (zero, identity, negated, wrong RoPE sign) that the checker must reject.
  * The DaisyChain-Train transformer.js page, function ``backward``: the batched causal
    multi-head form (keys tj <= ti) and the Wo linear backward convention.

All arithmetic is numpy float64 on values upcast from the exact stored inputs.
Module map:
  specs      single-vector specs as the API page states them (softmax, rope, rmsnorm,
             scaled dot, single-head attention Q/K/V backward)
  attention  batched multi-head / grouped-query / causal attention forward and backward
  layer      linear, row-wise RoPE and RMSNorm, one layer's backward and the stack
  verify     central differences, the gradient checker, the wrong backwards, run_all_checks
"""

from . import specs, attention, layer, verify  # noqa: F401
