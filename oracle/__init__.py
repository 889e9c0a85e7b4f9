"""fp64 CPU oracle for the fused MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never calls it, and it imports nothing from the product:
the two share no code.  The only thing both sides consume is the seeded input
data produced by the separate ``synth`` module.

Sources (web pages; citations give the page title and the section):
  * "Fused MoE kernel on Triton: 5 launches vs 24" (ai-manual.ru), section
    "Fused kernel: one operation instead of twenty-four": the layer is top-k
    routing weights, dispatch of tokens to the chosen experts, computation on
    every engaged expert, and aggregation of expert outputs with the routing
    weights.
  * "llama.cpp: fusing shared experts into MMVQ" (ai-manual.ru), section
    "Shared experts in MoE: what they are and why they exist": a router picks
    the top-k experts per token and only those compute; shared experts are
    active for every token whatever the router decides; section "What fusing
    gives computationally": fusion moves data differently but does not change
    the mathematics, so the oracle is the plain, unfused definition.

Readings where the pages are silent (each is listed with its reason in the
repository's design notes): SwiGLU experts without biases; softmax over all E
logits; top-k chosen on the logits, ties to the lower expert index; the k
selected probabilities renormalised to sum to 1; shared experts added with
weight 1; optional router bias added to the logits.

Modules:
  formats -- decoding of the stored input formats (bf16, fp16, Q4_0, Q8_0, fp8 E4M3)
  moe     -- vectorised fp64 reference (numpy), including the budgeted
             channel-sparse experts
  loops   -- pure-Python brute force for tiny shapes
"""
from . import formats, moe, loops  # noqa: F401
from .moe import (  # noqa: F401
    router_logits, softmax, select_topk, renormalize, route, near_ties,
    silu, swiglu_ffn, moe_forward, moe_forward_tokens, dispatch, dense_gate_matrix,
    select_channels, masked_swiglu, moe_forward_channel_sparse,
)
from .formats import (  # noqa: F401
    bf16_to_f64, f16_to_f64, q4_0_decode, q4_0_decode_matrix, q8_0_decode, q8_0_matrix, fp8_e4m3_to_f64,
    fp8_e4m3_decode, fp8_e4m3_matrix, weights_to_f64, decode_inputs,
    decode_workload_inputs,
)
from .moe import padded_rows  # noqa: F401
