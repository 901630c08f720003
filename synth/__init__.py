"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the benchmark.

This module draws random numbers and rounds them to the storage precision a workload
names (fp32, or bf16 by round-to-nearest-even from fp32). It holds none of the
backward pass's arithmetic: no softmax, no rotation, no normalisation, no products.
Tensors that a workload derives from a forward pass (row log-sum-exp, saved softmax
weights, normed activations) are not produced here; the caller obtains them from the
oracle (tests) or from the library's own forward helpers (benchmark).

Every array is returned as float32 (bf16 values are float32 arrays holding exactly
representable bf16 values) plus, for bf16, the raw 16-bit patterns for upload.
"""

from .gen import (  # noqa: F401
    bf16_bits,
    bf16_round,
    normal,
    uniform,
    Workload,
    WORKLOADS,
    tiny_inputs,
    decode_gqa_inputs,
    causal_inputs,
    layer_inputs,
    layer_upstream_grad,
    long_causal_inputs,
    attention_inputs,
    layernorm_inputs,
    relu2_inputs,
    ffn_inputs,
    block_inputs,
    rms_block_inputs,
)
