"""Seeded full-size inputs generated directly on the GPU with torch's RNG.

Same recipes as synthetic.workloads (which draws on the host with NumPy),
for sizes where host generation would dominate a test or the bench: weights
of the 32-layer stack, and logits over a 128256-token vocabulary for
thousands of rows.  Values are rounded to bf16 by the dtype conversion
(round to nearest even).  No method arithmetic lives here.
"""

import math

import torch

from .workloads import RANK, _exact_scale


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn(shape, std, seed, device="cuda", dtype=torch.bfloat16):
    g = _gen(seed, device)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def projection_weights(K, N, seed, r=RANK, device="cuda"):
    """(w [N,K], lora_a [r,K], lora_b [N,r]) bf16: N(0,1/K), N(0,1/K), N(0,1/r)."""
    return (randn((N, K), 1.0 / math.sqrt(K), seed, device),
            randn((r, K), 1.0 / math.sqrt(K), seed + 1, device),
            randn((N, r), 1.0 / math.sqrt(r), seed + 2, device))


def layer_weights(shapes, seed, r=RANK, device="cuda"):
    """{name: (w, a, b)} for one layer's projections ((name, K, N), ...)."""
    out = {}
    for i, (name, K, N) in enumerate(shapes):
        out[name] = projection_weights(K, N, seed + 10 * i, r, device)
    return out


def verify_logits(B, L, V, seed, kind="normal", target_sigma=3.0, draft_sigma=1.0, has_bonus=False,
                  device="cuda", dtype=torch.bfloat16, zipf_slope=1.1):
    """Target [B, L+has_bonus, V] and draft [B, L, V] logits (same recipes as the host generator)."""
    g = _gen(seed, device)
    rows_t = L + (1 if has_bonus else 0)
    if kind == "normal":
        z = torch.randn((B, rows_t, V), generator=g, device=device, dtype=torch.float32) * target_sigma
        d = z[:, :L, :] + torch.randn((B, L, V), generator=g, device=device, dtype=torch.float32) * draft_sigma
    elif kind == "zipf":
        z = torch.empty((B, rows_t, V), device=device, dtype=torch.float32)
        d = torch.empty((B, L, V), device=device, dtype=torch.float32)
        for b in range(B):  # per-sequence to bound the argsort working set
            ranks = torch.argsort(torch.rand((rows_t, V), generator=g, device=device), dim=-1).float() + 1.0
            base = -zipf_slope * torch.log(ranks)
            z[b] = base + torch.randn((rows_t, V), generator=g, device=device) * draft_sigma
            d[b] = base[:L] + torch.randn((L, V), generator=g, device=device) * draft_sigma
    else:
        raise ValueError(kind)
    return z.to(dtype).contiguous(), d.to(dtype).contiguous()


def random_tokens(B, L, V, seed, device="cuda"):
    """Uniformly random token ids (int32) -- filler drafts for rows a test does not inspect."""
    g = _gen(seed, device)
    return torch.randint(0, V, (B, L), generator=g, device=device, dtype=torch.int32)


def lm_head_tensors(B, L, V, K, seed, has_bonus=False, kind="normal", logit_sigma=3.0, draft_noise=0.3,
                    device="cuda"):
    """The LM head's inputs on the device, same recipes as synthetic.workloads.lm_head_inputs:
    (hidden [B (L+nb) + B L, K] bf16, w [V, K] bf16, tokens [B, L] int32, uniforms [B, L+1] float32)."""
    g = _gen(seed, device)
    nb = 1 if has_bonus else 0
    if kind == "normal":
        ht = torch.randn((B, L + nb, K), generator=g, device=device)
        hd = ht[:, :L] + torch.randn((B, L, K), generator=g, device=device) * draft_noise
        w = (torch.randn((V, K), generator=g, device=device) * (logit_sigma / math.sqrt(K))).to(torch.bfloat16)
    elif kind == "exact":
        ht = torch.randint(-3, 4, (B, L + nb, K), generator=g, device=device).float()
        hd = ht[:, :L] + torch.randint(-1, 2, (B, L, K), generator=g, device=device).float()
        w = (torch.randint(-2, 3, (V, K), generator=g, device=device).float() * _exact_scale(K)).to(torch.bfloat16)
    else:
        raise ValueError(kind)
    hidden = torch.cat([ht.reshape(B * (L + nb), K), hd.reshape(B * L, K)]).to(torch.bfloat16).contiguous()
    tokens = torch.randint(0, V, (B, L), generator=g, device=device, dtype=torch.int32)
    uniforms = torch.rand((B, L + 1), generator=g, device=device, dtype=torch.float32)
    return hidden, w.contiguous(), tokens, uniforms
