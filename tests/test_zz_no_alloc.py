"""uno_block_verify_noalloc: block verification with the library's own scratch
array instead of a caller workspace (for callers that cannot allocate).

Through the C ABI: two calls in a row on one GPU, the second on a smaller
problem (the array keeps the first call's contents), each compared with
uno_block_verify on the same inputs (the same kernels: bitwise equal), and
the bench's full size; a problem past the array is rejected before anything
runs.
"""

import numpy as np
import pytest
import torch

import lossless_speculative_drafting_amd as uno
from gpu_util import say, to_host
from synthetic import device as sdev

CASES = [  # B, L, V, has_bonus, T, kind
    (32, 16, 128256, False, 1.0, "normal"),   # the bench's verify call
    (3, 5, 1000, True, 0.7, "normal"),        # then a smaller one: stale scratch from the first
    (256, 32, 128256, False, 0.6, "zipf"),    # the largest workload's verify call (16 MiB of scratch)
    (1, 16, 128256, False, 1.0, "normal"),    # one sequence (the split tail)
]


def _inputs(B, L, V, has_bonus, kind, seed):
    z, d = sdev.verify_logits(B, L, V, seed=seed, kind=kind, has_bonus=has_bonus)
    x = sdev.random_tokens(B, L, V, seed + 1)
    u = torch.rand((B, L + 1), generator=torch.Generator(device="cuda").manual_seed(seed + 2), device="cuda")
    # draft tokens drawn on the GPU from the draft logits, so acceptance is realistic
    x = uno.draft_sample(d, u[:, :L].contiguous(), 1.0)
    return z, d, x, u


def _outputs(B, L):
    return (torch.full((B,), -9, dtype=torch.int32, device="cuda"),
            torch.full((B, L + 1), -9, dtype=torch.int32, device="cuda"),
            torch.full((B,), -9, dtype=torch.int32, device="cuda"))


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_verifier_on_consecutive_calls():
    for i, (B, L, V, has_bonus, T, kind) in enumerate(CASES):
        say("noalloc verify", B, L, V, has_bonus, T, kind)
        z, d, x, u = _inputs(B, L, V, has_bonus, kind, 100 + i)
        ref = uno.block_verify(z, d, x, u, T, has_bonus)
        out = _outputs(B, L)
        uno.block_verify(z, d, x, u, T, has_bonus, outputs=out, noalloc=True)
        torch.cuda.synchronize()
        for a, b in zip(ref, out):
            np.testing.assert_array_equal(to_host(a), to_host(b))
        print(f"  mean emitted {to_host(out[2]).mean():.2f}", flush=True)


@pytest.mark.gpu
def test_noalloc_rejects_problems_past_its_scratch():
    lib = uno.library()
    cap = lib.uno_block_verify_noalloc_max_bytes()
    assert cap == 32 << 20
    B, L, V = 4096, 16, 128256
    assert lib.uno_block_verify_workspace_size(B, L, V, 0) > cap
    say("noalloc rejects", B, L, V)
    z = torch.zeros((1, L, V), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((B, L), dtype=torch.int32, device="cuda")
    u = torch.zeros((B, L + 1), dtype=torch.float32, device="cuda")
    out = _outputs(B, L)
    with pytest.raises(uno.UnoError) as e:
        uno.block_verify(z, z, x, u, 1.0, False, outputs=out, noalloc=True)
    assert e.value.status == 2 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out[0] == -9).all()), "a rejected call enqueues nothing"
