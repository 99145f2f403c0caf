"""MI355X-native hot path of Uno's draft+verify step.

Python binding over libuno.so (hand-written HIP for gfx950):

* gated_lora_fwd  -- y = x W_AR + g * (alpha/r) * (x A) B on a mixed batch of
                     draft (g = 1) and verify (g = 0) rows;
* block_verify    -- lossless speculative verification of drafted blocks;
* lm_head_verify  -- the LM head with the verification statistics in its
                     epilogue, then the same verification (no logit rows
                     written unless asked for);
* draft_sample    -- parallel inverse-CDF proposal of draft tokens;
* tree_verify     -- verification of candidate prefix trees (the tree sampler);
* philox_uniforms -- the counter-based uniforms both consume;
* rmsnorm, silu_mul, residual_add -- glue of the synthetic layer stack.

Importing the package loads the shared library; there is no CPU fallback.
"""

from ._lib import (  # noqa: F401
    UNO_BF16,
    UNO_F32,
    RowPlan,
    UnoError,
    Workspace,
    block_verify,
    block_verify_early_workspace_size,
    block_verify_workspace_size,
    draft_sample,
    draft_sample_workspace_size,
    gated_gemm,
    gated_gemm_grouped,
    gated_gemm_residual,
    gated_gemm_swiglu,
    gated_lora_fwd,
    gated_lora_workspace_size,
    header_symbols,
    library,
    lm_head_verify,
    lm_head_verify_workspace_size,
    lora_down,
    lora_t_size,
    philox_uniforms,
    residual_add,
    residual_rmsnorm,
    rmsnorm,
    silu_mul,
    status_string,
    swiglu_pack,
    tree_verify,
    tree_verify_workspace_size,
)
from .stack import GatedLoraStack  # noqa: F401
