"""Parallel draft proposal (inverse CDF over q = softmax(d / T)) vs the oracle."""

import numpy as np
import pytest
import torch

import lossless_speculative_drafting_amd as uno
import oracle
from gpu_util import say, to_dev, to_host
from parity import compare_samples
from synthetic import device as sdev, verify_inputs


@pytest.mark.gpu
@pytest.mark.parametrize("B,L,V,dtype,T", [(3, 5, 999, "f32", 1.0), (8, 4, 4096, "bf16", 0.6),
                                           (2, 3, 1, "bf16", 1.0), (50, 70, 64, "f32", 1.0),
                                           (2, 2, 300000, "bf16", 1.0)])  # segment sums past the LDS staging
def test_draft_sample_small(B, L, V, dtype, T):
    _, d = verify_inputs(B, L, V, seed=B + L + V, dtype=dtype)
    u = oracle.philox_uniforms(0, 1, 0, B * L).reshape(B, L)
    say("draft sample", B, L, V, dtype, T)
    tok = to_host(uno.draft_sample(to_dev(d, dtype), to_dev(u, "f32"), T))
    ref = oracle.draft_sample(d, u, T)
    exact, excused, fails = compare_samples(tok.reshape(-1), ref.reshape(-1), d.reshape(-1, V), u.reshape(-1), T)
    print(f"  exact {exact} excused {excused}", flush=True)
    assert not fails, fails[:5]


@pytest.mark.gpu
def test_draft_sample_full_vocab():
    B, L, V = 32, 16, 128256
    say("draft sample full vocab", B, L, V)
    _, dt = sdev.verify_logits(B, L, V, 1005, draft_sigma=1.0)
    u = oracle.philox_uniforms(0, 1, 0, B * L).reshape(B, L)
    tok = to_host(uno.draft_sample(dt, to_dev(u, "f32"), 1.0)).reshape(-1)
    torch.cuda.synchronize()
    d = to_host(dt).reshape(B * L, V)
    ref = oracle.draft_sample(d, u.reshape(-1), 1.0)
    exact, excused, fails = compare_samples(tok, ref, d, u.reshape(-1), 1.0)
    print(f"  exact {exact} excused {excused}", flush=True)
    assert not fails, fails[:5]
    assert excused <= 5
