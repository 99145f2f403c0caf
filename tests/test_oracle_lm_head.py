"""Pins for the LM-head oracle (CPU only): its bf16 rounding against torch's
float32 -> bfloat16 conversion and closed forms, the head's orientation
through a permutation matrix, and the stacked row order through a head that
returns the hidden states themselves."""

import numpy as np
import pytest
import torch

from oracle import lm_head
from oracle.verify import block_verify


def test_bf16_round_matches_torch_on_binary32_values():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 10,
        rng.standard_normal(2000).astype(np.float32) * np.float32(1e-39),  # binary32 subnormals
        (rng.random(2000).astype(np.float32) * np.float32(3.4e38)),           # near the top, incl. overflow
        np.array([0.0, -0.0, 1.0, -1.0], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(lm_head.bf16_round(x), ref)


def test_bf16_round_ties_to_even():
    # spacing 2^-7 on [1, 2): midpoints go to the even neighbour
    got = lm_head.bf16_round([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 1 + 2**-8 + 2**-40])
    np.testing.assert_array_equal(got, [1.0, 1 + 2**-6, -1.0, 1 + 2**-7])
    assert lm_head.bf16_round([2.0**-133 * 1.5])[0] == 2.0**-132   # smallest spacing, tie to even
    assert np.isinf(lm_head.bf16_round([3.4e38])[0])


def test_head_orientation_by_permutation():
    rng = np.random.default_rng(1)
    K = 24
    perm = rng.permutation(K)
    w = np.zeros((K, K))
    w[np.arange(K), perm] = 1.0          # logit v reads hidden column perm[v]
    h = lm_head.bf16_round(rng.standard_normal((5, K)))
    np.testing.assert_array_equal(lm_head.lm_head_logits(h, w), h[:, perm])


def test_rank_one_head_is_the_outer_product():
    h = np.array([[1.5], [-2.0], [0.25]])
    w = np.array([[2.0], [-0.5], [3.0], [0.0]])
    np.testing.assert_array_equal(lm_head.lm_head_logits(h, w), lm_head.bf16_round(h @ w.T))
    np.testing.assert_array_equal(lm_head.lm_head_logits(h, w)[0], [3.0, -0.75, 4.5, 0.0])


@pytest.mark.parametrize("has_bonus", [False, True])
def test_stacked_rows_are_target_then_draft(has_bonus):
    """With the identity head the logits are the hidden rows, so verification
    of the stacked rows must equal block_verify on the arrays cut by hand."""
    rng = np.random.default_rng(3)
    B, L, V = 3, 4, 16
    nb = 1 if has_bonus else 0
    z = lm_head.bf16_round(rng.standard_normal((B, L + nb, V)) * 2)
    d = lm_head.bf16_round(z[:, :L] + rng.standard_normal((B, L, V)) * 0.5)
    hidden = np.concatenate([z.reshape(B * (L + nb), V), d.reshape(B * L, V)])
    x = rng.integers(0, V, (B, L))
    u = rng.random((B, L + 1))
    got = lm_head.lm_head_verify(hidden, np.eye(V), x, u, temperature=0.8, has_bonus=has_bonus)
    ref = block_verify(z, d, x, u, temperature=0.8, has_bonus=has_bonus)
    for k in ("n_accepted", "out_tokens", "n_emitted", "redraw_row"):
        np.testing.assert_array_equal(got[k], ref[k])
    np.testing.assert_array_equal(got["accept_prob"], ref["accept_prob"])
    # the other order verifies something else
    swapped = np.concatenate([d.reshape(B * L, V), z.reshape(B * (L + nb), V)])
    if not has_bonus:
        alt = lm_head.lm_head_verify(swapped, np.eye(V), x, u, temperature=0.8)
        assert not np.array_equal(alt["accept_prob"], ref["accept_prob"])
