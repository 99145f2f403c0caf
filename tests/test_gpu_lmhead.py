"""The LM head with the verification statistics in its epilogue, on the GPU.

* Exact inputs (small integers, so every fp32 sum of products is exact and
  the bf16 logits are the oracle's bit for bit): the outputs must equal the
  fp64 oracle's (LM head, then block verification) under the same rule as
  the verifier's own tests (tests/parity.py: ties within 1e-6 of the uniform
  are excused and counted), and the stored logits must equal the oracle's.
  Drafts are drawn with the oracle's inverse CDF from the oracle's draft
  distribution.
* Normal inputs: both modes (logits stored, or redraw rows recomputed) must
  agree bit for bit; the fused outputs and those of uno_block_verify on the
  stored logits must each match the oracle run on those stored logits under
  the tie rule (the two sum their exponentials in different orders, so a
  decision may differ between them only where a uniform lies within about
  1e-7 of an acceptance probability or CDF boundary); the stored logits are
  checked against the oracle's to the bf16 GEMM tolerance.
* The redraw rows recomputed when no logits are stored are bitwise the
  stored logit rows, at shapes where the planner's cheapest tile for the
  recompute would be a two-K-group one, and with such a tile forced.
* The bench's size (32 sequences x 16 drafted positions, V = 128256,
  K = 4096): both modes agree, and four sampled sequences match the oracle.
"""

import numpy as np
import pytest
import torch

import lossless_speculative_drafting_amd as uno
import oracle
from gpu_util import say, to_dev, to_host
from parity import BF16_TOL, compare_verify, floored_rel_err
from synthetic import device as sdev
from synthetic import lm_head_inputs


def _drafts(d, T, seed=0):
    B, L, V = d.shape
    u = oracle.philox_uniforms(seed, 1, 0, B * L).reshape(B, L)
    return np.stack([oracle.draft_sample(d[:, i, :], u[:, i], T) for i in range(L)], axis=1).astype(np.int32)


def _run(hidden, w, x, u, T, has_bonus, store):
    rows, V = hidden.shape[0], w.shape[0]
    logits = torch.empty((rows, V), dtype=torch.bfloat16, device="cuda") if store else None
    out = uno.lm_head_verify(hidden, w, x, u, T, has_bonus, logits=logits)
    torch.cuda.synchronize()
    return tuple(to_host(t) for t in out), logits


CASES = [  # B, L, V, K, has_bonus, T
    (3, 5, 1000, 256, False, 1.0),   # V ragged over the 256-column tiles
    (4, 7, 997, 128, True, 0.7),     # V % 8 != 0: logit rows not 16-byte aligned
    (2, 16, 4096, 512, True, 1.0),
    (1, 1, 256, 64, False, 1.3),     # one position, one tile
    (37, 4, 600, 64, True, 1.0),     # many sequences
    (2, 3, 262400, 64, True, 1.0),   # redraw rows past the one-workgroup tail's LDS staging
]


@pytest.mark.gpu
@pytest.mark.parametrize("store", [False, True])
@pytest.mark.parametrize("B,L,V,K,has_bonus,T", CASES)
def test_exact_inputs_match_the_oracle(B, L, V, K, has_bonus, T, store):
    inp = lm_head_inputs(B, L, V, K, seed=B * 7 + L + V + K, has_bonus=has_bonus, kind="exact")
    ref_logits = oracle.lm_head.lm_head_logits(inp["hidden"], inp["w"])
    z, d = oracle.lm_head.split_rows(ref_logits, B, L, has_bonus)
    x = _drafts(d, T)
    u = oracle.philox_uniforms(0, 0, 0, B * (L + 1)).reshape(B, L + 1)
    say("lm_head exact", B, L, V, K, has_bonus, T, "store" if store else "recompute")
    gpu, logits = _run(to_dev(inp["hidden"], "bf16"), to_dev(inp["w"], "bf16"), to_dev(x, "i32"),
                       to_dev(u, "f32"), T, has_bonus, store)
    ref = oracle.block_verify(z, d, x, u.astype(np.float64), T, has_bonus)
    exact, excused, fails = compare_verify(gpu, ref, z, d, u.astype(np.float64), T, has_bonus)
    print(f"  exact {exact} excused ties {excused} failures {len(fails)}", flush=True)
    assert not fails, fails[:5]
    assert excused <= 1
    if store:
        np.testing.assert_array_equal(to_host(logits), ref_logits)


@pytest.mark.gpu
@pytest.mark.parametrize("tail", ["default", "fused"])
@pytest.mark.parametrize("B,L,V,K,has_bonus,T", [(8, 16, 8192 + 96, 512, True, 1.0), (5, 9, 3000, 256, False, 0.8)])
def test_modes_agree_bitwise_and_match_the_unfused_verifier(B, L, V, K, has_bonus, T, tail, monkeypatch):
    if tail != "default":
        monkeypatch.setenv("UNO_VERIFY_TAIL", tail)
    inp = lm_head_inputs(B, L, V, K, seed=V + K, has_bonus=has_bonus, kind="normal")
    hidden, w = to_dev(inp["hidden"], "bf16"), to_dev(inp["w"], "bf16")
    nb = 1 if has_bonus else 0
    nt = B * (L + nb)
    u = to_dev(inp["uniforms"], "f32")
    # drafts drawn on the GPU from the stored draft logits (GPU-only comparison)
    say("lm_head modes", B, L, V, K, has_bonus)
    logits = torch.empty((hidden.shape[0], V), dtype=torch.bfloat16, device="cuda")
    uno.lm_head_verify(hidden, w, to_dev(inp["tokens"], "i32"), u, T, has_bonus, logits=logits)
    du = torch.rand((B, L), generator=torch.Generator(device="cuda").manual_seed(5), device="cuda")
    x = uno.draft_sample(logits[nt:].view(B, L, V), du, T)
    store, _ = _run(hidden, w, x, u, T, has_bonus, True)
    recompute, _ = _run(hidden, w, x, u, T, has_bonus, False)
    for a, b in zip(store, recompute):
        np.testing.assert_array_equal(a, b)
    out = uno.block_verify(logits[:nt].view(B, L + nb, V), logits[nt:].view(B, L, V), x, u, T, has_bonus)
    torch.cuda.synchronize()
    unfused = tuple(to_host(t) for t in out)
    lg = to_host(logits).astype(np.float64)
    z, d = lg[:nt].reshape(B, L + nb, V), lg[nt:].reshape(B, L, V)
    uh = to_host(u).astype(np.float64).reshape(B, L + 1)
    ref = oracle.block_verify(z, d, to_host(x), uh, T, has_bonus)
    for name, res in (("fused", store), ("unfused", unfused)):
        exact, excused, fails = compare_verify(res, ref, z, d, uh, T, has_bonus)
        print(f"  {name}: exact {exact} excused ties {excused}", flush=True)
        assert not fails, (name, fails[:5])
        assert excused <= 1
    acc = store[0]
    print(f"  mean accepted {acc.mean():.2f} of {L}", flush=True)
    rows = np.array([0, nt - 1, nt, hidden.shape[0] - 1, nt // 2])
    ref = oracle.lm_head.lm_head_logits(inp["hidden"][rows], inp["w"])
    assert floored_rel_err(to_host(logits)[rows], ref) <= BF16_TOL


@pytest.mark.gpu
def test_bench_size_modes_agree_and_sampled_sequences_match_the_oracle():
    B, L, V, K, has_bonus, T = 32, 16, 128256, 4096, False, 1.0
    say("lm_head full size", B, L, V, K)
    hidden, w, x, u = sdev.lm_head_tensors(B, L, V, K, seed=77, has_bonus=has_bonus, kind="exact")
    seqs = [0, 7, 19, 31]
    rows_of = lambda s: list(range(s * L, (s + 1) * L)) + list(range(B * L + s * L, B * L + (s + 1) * L))
    rows = np.array([r for s in seqs for r in rows_of(s)])
    h_host = to_host(hidden)[rows]
    w_host = to_host(w)
    ref_logits = oracle.lm_head.lm_head_logits(h_host, w_host)
    z = np.stack([ref_logits[i * 2 * L:i * 2 * L + L] for i in range(len(seqs))])
    d = np.stack([ref_logits[i * 2 * L + L:(i + 1) * 2 * L] for i in range(len(seqs))])
    xs = _drafts(d, T)
    x[seqs] = to_dev(xs, "i32")
    store, logits = _run(hidden, w, x, u, T, has_bonus, True)
    recompute, _ = _run(hidden, w, x, u, T, has_bonus, False)
    for a, b in zip(store, recompute):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(to_host(logits[torch.from_numpy(rows).cuda()]), ref_logits)
    uh = to_host(u)[seqs].astype(np.float64)
    ref = oracle.block_verify(z, d, xs, uh, T, has_bonus)
    gpu = tuple(a[seqs] for a in store)
    exact, excused, fails = compare_verify(gpu, ref, z, d, uh, T, has_bonus)
    print(f"  sampled: exact {exact} excused {excused}; mean accepted (all) {store[0].mean():.2f}", flush=True)
    assert not fails, fails[:5]


@pytest.mark.gpu
@pytest.mark.parametrize("B,L,V,K,has_bonus,tile", [
    (32, 4, 32000, 4096, False, None),            # 64 recomputed rows: the planner's two-K-group pick
    (64, 2, 32000, 4096, True, None),
    (24, 3, 32000, 4096, False, "128x128b4kg2"),  # a forced two-K-group tile is not taken either
])
def test_recomputed_redraw_rows_are_the_stored_logits(B, L, V, K, has_bonus, tile, monkeypatch):
    """Without stored logits, the 2 B redraw rows are recomputed by the LM-head GEMM into the
    last 2 B V bf16 values of the workspace (row 2s: the target row of sequence s's redraw,
    2s + 1: its draft row, for a residual redraw); they must be the bits of the stored logits."""
    if tile:
        monkeypatch.setenv("UNO_GEMM_TILE", tile)
    say("lm_head recompute rows", B, L, V, K, has_bonus, tile)
    hidden, w, x, u = sdev.lm_head_tensors(B, L, V, K, seed=B + V, has_bonus=has_bonus, kind="normal")
    nb = 1 if has_bonus else 0
    nt = B * (L + nb)
    store, logits = _run(hidden, w, x, u, T=1.0, has_bonus=has_bonus, store=True)
    ws = uno.Workspace(hidden.device)
    out = uno.lm_head_verify(hidden, w, x, u, 1.0, has_bonus, logits=None, workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip(store, (to_host(t) for t in out)):
        np.testing.assert_array_equal(a, b)
    need = uno.lm_head_verify_workspace_size(B, L, V, K, has_bonus)
    rc_bytes = (2 * B * V * 2 + 255) // 256 * 256
    rc = ws.buf[need - rc_bytes:need - rc_bytes + 2 * B * V * 2].view(torch.int16).view(2 * B, V)
    lg = logits.view(torch.int16)
    n_acc, _, n_emit = store
    checked = 0
    for s in range(B):
        if n_acc[s] < L:   # residual redraw at position n_acc: target and draft rows
            j = int(n_acc[s])
            assert torch.equal(rc[2 * s], lg[s * (L + nb) + j]), s
            assert torch.equal(rc[2 * s + 1], lg[nt + s * L + j]), s
            checked += 1
        elif has_bonus:   # bonus draw from the target row L
            assert torch.equal(rc[2 * s], lg[s * (L + nb) + L]), s
            checked += 1
    print(f"  redraw rows checked: {checked} of {B} sequences", flush=True)
    assert checked >= 4
