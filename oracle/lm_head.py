"""The LM head followed by block verification -- TEST INFRASTRUCTURE ONLY.

What is computed.  The sampler of the pages ("The Ψ-Spec Sampler" on the
aifromscratch.in page; "What 'lossless' means here" on the cctest.ai page)
compares, at every drafted position, the AR model's next-token distribution
with the one the drafting pathway sampled from.  Both are softmaxes of the
model's output logits, which the model's last linear layer (the LM head)
forms from each row's final hidden state.

Readings taken where the pages are silent:

* the head is one linear map shared by target and draft rows,
  ``z = h W^T`` with ``w`` stored ``[V, K]`` (``nn.Linear`` layout); the
  pages put the LoRA adapter on the transformer layers' projections, not on
  the head;
* the logits are held in bf16, the storage type of the verifier's inputs at
  the workloads: each logit is the exact product rounded once to the nearest
  bf16 value, ties to even (``bf16_round``);
* the rows come stacked as the library takes them: the target rows of every
  sequence (``L + has_bonus`` each), then the draft rows (``L`` each).

Everything after the head is ``oracle.verify.block_verify``.
"""

import numpy as np

from .verify import block_verify


def bf16_round(x):
    """Round each value to the nearest bfloat16 number, ties to even, in fp64.

    bfloat16 keeps 8 significant bits and the exponent range of binary32:
    a normal value m * 2^e (0.5 <= |m| < 1) becomes rint(m * 2^8) * 2^(e - 8);
    below 2^-126 the spacing is fixed at 2^-133; past the largest finite
    bfloat16 value the result is +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    normal = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    sub = np.rint(np.ldexp(x, 133)) * 2.0 ** -133
    y = np.where(np.abs(x) < 2.0 ** -126, sub, normal)
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127
    return np.where(np.abs(y) > big, np.copysign(np.inf, x), y)


def lm_head_logits(hidden, w):
    """bf16-rounded logits ``[rows, V]`` (float64 values) of ``hidden [rows, K]``."""
    h = np.asarray(hidden, dtype=np.float64)
    W = np.asarray(w, dtype=np.float64)
    if h.ndim != 2 or W.ndim != 2 or h.shape[1] != W.shape[1]:
        raise ValueError("hidden must be [rows, K] and w must be [V, K]")
    return bf16_round(h @ W.T)


def split_rows(logits, B, L, has_bonus=False):
    """Stacked rows -> (target [B, L + has_bonus, V], draft [B, L, V])."""
    nb = 1 if has_bonus else 0
    z = np.asarray(logits)
    nt = B * (L + nb)
    if z.shape[0] != nt + B * L:
        raise ValueError("expected B (L + has_bonus) + B L rows")
    return z[:nt].reshape(B, L + nb, -1), z[nt:].reshape(B, L, -1)


def lm_head_verify(hidden, w, draft_tokens, uniforms, temperature=1.0, has_bonus=False):
    """Block verification on the logits of the stacked hidden rows; returns
    ``block_verify``'s dict."""
    x = np.asarray(draft_tokens)
    B, L = x.shape
    z, d = split_rows(lm_head_logits(hidden, w), B, L, has_bonus)
    return block_verify(z, d, x, uniforms, temperature=temperature, has_bonus=has_bonus)
