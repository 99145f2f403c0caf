"""Plain fp64 CPU oracle for the Uno hot path -- TEST INFRASTRUCTURE ONLY.

This package states, slowly and in double precision, what the GPU library
computes, so that the library can be checked against it.  It is not part of
the product: only the test suite, the smoke check in ``__graft_entry__`` and
the CPU-baseline leg of ``bench.py`` may import it.  It shares no code,
constants, tables or helpers with the HIP library under
``lossless_speculative_drafting_amd/`` and imports nothing from it.

Sources.  The method is described on five web pages about *Unlocking
Lossless Speedups in LLMs via Discrete Diffusion* ("Uno"):

* "Unlocking Lossless Speedups in LLMs via Discrete Diffusion -- explained
  simply" (aifromscratch.in), sections "Two Decoupled Weight Sets" and
  "The Ψ-Spec Sampler";
* "Uno Uses Discrete Diffusion to Accelerate LLMs Without Loss"
  (cctest.ai), sections "How Uno works" and "What 'lossless' means here";
* "Unlocking Lossless Speedups in LLMs via Discrete Diffusion" (aiany.app),
  section "Key Findings".

The pages give the constants (LoRA rank 128, alpha 256), the gating rule
(draft pathway = AR weights + LoRA, verify pathway = AR weights only) and the
sampler contract (draft a block in parallel, rejection-sample it against the
AR model in the style of speculative decoding, keep the longest accepted
prefix, preserve the AR distribution exactly).  They print no formula, code
or worked example, so every step below is the standard textbook reading of
that contract; each function names the reading it takes.

Modules
-------
``philox``      Philox4x32-10 words and 24-bit uniforms (Salmon et al., SC'11).
``gated_lora``  y = x W_AR + g (alpha/r) (x A) B in fp64.
``verify``      softmax, acceptance test, first-rejection scan, residual
                resampling, emit, and inverse-CDF draft sampling.
``stack``       the weightless RMSNorm / SiLU-gate glue used between the
                projections of the synthetic layer stack.
``lm_head``     bf16 logits of the LM head and block verification on them.
``tree``        verification of a candidate prefix tree (the tree sampler).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against something other than itself (a library special case, brute force,
exact enumeration, closed forms or a chi-square test).
"""

from .philox import philox4x32_10, philox_words, philox_uniforms, words_to_uniform
from .gated_lora import gated_lora
from .verify import (
    log_softmax,
    acceptance_probability,
    inverse_cdf,
    block_verify,
    residual_weights,
    draft_sample,
)
from . import stack
from . import lm_head
from . import tree

__all__ = [
    "philox4x32_10",
    "philox_words",
    "philox_uniforms",
    "words_to_uniform",
    "gated_lora",
    "log_softmax",
    "acceptance_probability",
    "inverse_cdf",
    "block_verify",
    "residual_weights",
    "draft_sample",
    "stack",
    "lm_head",
    "tree",
]
