"""CPU oracle for the canvas denoise pass -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain reference that the HIP path is checked
against.  Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import it; the product path never does, and it shares no code with
the HIP library (the two meet only through the seeded inputs of ``synth``).

Arithmetic is float64 throughout.  In bf16 workloads values are rounded to
bf16 exactly where the GPU path stores them in bf16 (weights, prompt KV, the
normalised GEMM inputs, q/k/v after RoPE, the attention output, the GeGLU
output, the final hidden state); everything else (residual stream, scores,
softmax, router logits, gates, logits, confidence) stays in float64.

Sources, by the title of the page and the section:

* [HandsOn] "Hands-On with Diffusion Gemma: Another Gemma with a Diffusion
  Mechanism" -- sections "How Is This Different from Previous Models?" and
  "Detailed Specs".
* [4xFaster] "DiffusionGemma: The Diffusion Era Begins with 4x Faster Text
  Generation" -- sections "What is Diffusion and Why is it Coming to Text
  Generation Now?" and "DiffusionGemma's Technical Architecture".
* [ParadigmShift] "DiffusionGemma: Exploring the Paradigm Shift in
  Non-Autoregressive Language Modeling" -- sections "The Mechanics of
  Non-Autoregressive Generation" and "Analysis of Implications".
* [Experimental] "DiffusionGemma: Google's Experimental Diffusion LLM" --
  section "How Text Diffusion Actually Works".

Pinning.  Every function here is pinned by the ``-m "not gpu"`` tests against
closed forms, invariants, library routines or exhaustive enumeration (see
``tests/test_oracle_pins.py``).  Absolute values of whole multi-layer passes
are pinned only through those per-step pins: the pages print no worked
example of a pass.
"""
from .model import (  # noqa: F401
    OracleWeights, argmax_conf, attention_heads, canvas_attention, qkv_rope, Shadow, forward_hidden, bf16_bits_to_f64, bf16_round,
    denoise_pass, expert_ffn, gelu_tanh, generate_block, layer_forward, lm_logits,
    lock_count, lock_select, moe_block, rmsnorm, rope, route, softmax_attention,
)
