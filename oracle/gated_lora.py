"""Gated-LoRA projection in fp64 -- TEST INFRASTRUCTURE ONLY.

What is computed.  "Unlocking Lossless Speedups in LLMs via Discrete
Diffusion -- explained simply" (aifromscratch.in), section "Two Decoupled
Weight Sets": every layer keeps its frozen autoregressive weights and gains a
LoRA adapter of rank 128 with alpha 256; the draft pathway runs the AR weights
plus the adapter, the verification pathway runs the AR weights alone, and a
gate couples the two.  "Uno Uses Discrete Diffusion to Accelerate LLMs Without
Loss" (cctest.ai), section "How Uno works", describes the same split as an AR
foundation plus a lightweight diffusion drafting path.

Readings taken where the pages are silent:

* the LoRA update has the usual form ``(alpha/r) * (x A) B`` so the scale is
  256/128 = 2;
* the gate is one value per token row: 1 for a draft-block row, 0 for a
  verification row, so one mixed batch serves both pathways:

      y_m = x_m W_AR + g_m * (alpha/r) * (x_m A) B

* storage follows the ``nn.Linear`` convention used by the library:
  ``w`` is ``[N, K]`` (so ``W_AR = w.T``), ``a`` is ``[r, K]`` (so
  ``A = a.T``) and ``b`` is ``[N, r]`` (so ``B = b.T``).

Arithmetic is fp64 on the exact input values, with no intermediate rounding.
Rows with g = 0 are therefore ``x W_AR`` exactly as NumPy's fp64 matmul forms
it.
"""

import numpy as np


def gated_lora(x, w, a, b, gate, scale=2.0):
    """Return ``y`` ([M, N], float64) for one gated-LoRA projection.

    x    : [M, K] input rows
    w    : [N, K] frozen AR weight (W_AR = w.T)
    a    : [r, K] LoRA down-projection (A = a.T)
    b    : [N, r] LoRA up-projection (B = b.T)
    gate : [M] values in {0, 1}; 1 selects the draft pathway
    scale: alpha / r (2.0 for rank 128, alpha 256)
    """
    x = np.asarray(x, dtype=np.float64)
    W_AR = np.asarray(w, dtype=np.float64).T      # [K, N]
    A = np.asarray(a, dtype=np.float64).T         # [K, r]
    B = np.asarray(b, dtype=np.float64).T         # [r, N]
    g = np.asarray(gate)
    if x.ndim != 2 or W_AR.shape[0] != x.shape[1]:
        raise ValueError("x must be [M, K] and w must be [N, K]")
    if A.shape[0] != x.shape[1] or B.shape[0] != A.shape[1] or B.shape[1] != W_AR.shape[1]:
        raise ValueError("a must be [r, K] and b must be [N, r]")
    if g.shape != (x.shape[0],) or not np.all((g == 0) | (g == 1)):
        raise ValueError("gate must be a length-M vector of 0/1 values")

    y = x @ W_AR                                  # verify pathway: AR weights only
    draft = g.astype(bool)
    if np.any(draft):
        xd = x[draft]
        y[draft] = y[draft] + float(scale) * ((xd @ A) @ B)   # draft pathway adds the adapter
    return y
