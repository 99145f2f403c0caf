"""Glue between the projections of the synthetic layer stack -- TEST INFRASTRUCTURE ONLY.

The pages place a second (LoRA) pathway in every transformer layer
("Unlocking Lossless Speedups in LLMs via Discrete Diffusion -- explained
simply", aifromscratch.in, section "How It Works: The 'Uno' Architecture")
but say nothing about the rest of the layer.  The synthetic stack therefore
takes the plainest Llama-like chain with the attention mixing left out
(identity attention), and random, weightless normalisation:

    h  = rmsnorm(x)
    q, k, v = proj_q(h), proj_k(h), proj_v(h)     (k and v are computed, unused)
    x  = x + proj_o(q)
    h  = rmsnorm(x)
    x  = x + proj_down(silu(proj_gate(h)) * proj_up(h))

where every proj_* is one gated-LoRA projection.  These three helpers are
the non-projection steps, in fp64.
"""

import numpy as np

RMS_EPS = 1e-5


def rmsnorm(x, eps=RMS_EPS):
    """x / sqrt(mean(x**2) + eps) per row, with no learned weight."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def silu_mul(gate, up):
    """silu(gate) * up, with silu(t) = t / (1 + exp(-t))."""
    g = np.asarray(gate, dtype=np.float64)
    u = np.asarray(up, dtype=np.float64)
    return g / (1.0 + np.exp(-g)) * u


def residual_add(x, y):
    """x + y."""
    return np.asarray(x, dtype=np.float64) + np.asarray(y, dtype=np.float64)
