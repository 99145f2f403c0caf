"""Block verification on the GPU vs the fp64 oracle.

Accepted lengths, emitted tokens and counts must match exactly; the only
excused differences are ties within 1e-6 of the uniform (tests/parity.py),
which are counted and printed.  Drafts are drawn with the oracle's inverse
CDF from the draft distribution (Philox stream 1), uniforms come from the
oracle's Philox (stream 0), so both sides see identical inputs.
"""

import numpy as np
import pytest
import torch

import lossless_speculative_drafting_amd as uno
import oracle
from gpu_util import say, to_dev, to_host
from parity import compare_verify
from synthetic import WORKLOADS, device as sdev, verify_inputs


def _drafts(d, T, seed=0):
    B, L, V = d.shape
    u = oracle.philox_uniforms(seed, 1, 0, B * L).reshape(B, L)
    return np.stack([oracle.draft_sample(d[:, i, :], u[:, i], T) for i in range(L)], axis=1)


def _check(z, d, x, u, T, has_bonus, dtype, label, max_excused_frac=0.01):
    say("verify", label)
    out = uno.block_verify(to_dev(z, dtype), to_dev(d, dtype), to_dev(x, "i32"), to_dev(u, "f32"), T, has_bonus)
    torch.cuda.synchronize()
    gpu = tuple(to_host(t) for t in out)
    ref = oracle.block_verify(z, d, x, u, T, has_bonus)
    exact, excused, fails = compare_verify(gpu, ref, z, d, u, T, has_bonus)
    print(f"  {label}: exact {exact} excused ties {excused} failures {len(fails)}", flush=True)
    assert not fails, fails[:5]
    assert excused <= max(1, max_excused_frac * len(x))
    return gpu, ref


@pytest.mark.gpu
@pytest.mark.parametrize("path", ["default", "general"])
@pytest.mark.parametrize("has_bonus", [False, True])
def test_tiny_workload(has_bonus, path, monkeypatch):
    if path == "general":  # (V <= 1024 otherwise takes the one-wavefront-per-sequence kernel)
        monkeypatch.setenv("UNO_VERIFY_SMALL", "0")
    wl = WORKLOADS["tiny"]
    B, L, V, T = 2, wl.block, wl.vocab, 1.0
    z, d = verify_inputs(B, L, V, wl.seed, "normal", wl.target_sigma, wl.draft_sigmas[0], has_bonus, "f32")
    x = _drafts(d, T)
    u = oracle.philox_uniforms(0, 0, 0, B * (L + 1)).reshape(B, L + 1).astype(np.float64)
    _check(z, d, x, u, T, has_bonus, "f32", f"tiny bonus={has_bonus}")


CASES = [  # B, L, V, dtype, kind, sigma, T, bonus
    (37, 7, 1000, "bf16", "normal", 1.0, 1.0, False),
    (37, 7, 999, "bf16", "normal", 0.25, 0.6, True),      # V % 8 != 0: scalar-load path
    (16, 64, 4096, "bf16", "normal", 1.0, 1.0, False),    # longest block
    (9, 63, 520, "f32", "normal", 4.0, 1.0, True),        # longest block with a bonus row
    (64, 16, 2048, "bf16", "zipf", 0.5, 0.6, False),
    (5, 3, 1, "bf16", "normal", 1.0, 1.0, True),          # single-token vocabulary
    (300, 2, 17, "f32", "normal", 1.0, 2.0, False),       # many sequences, odd V
    (3, 4, 300000, "bf16", "normal", 1.0, 1.0, True),     # rows past the one-workgroup tail's LDS staging
    # one statistics chunk per row (96 x 17 rows): the pipelined loop's steps
    # of 2 x 2048 tokens -- one step then the plain tail, two steps (the loop
    # once, its last loads re-reading), three (the loop once, then the odd
    # step) -- and the bonus row's target-only form
    (96, 16, 6152, "bf16", "normal", 1.0, 1.0, True),
    (96, 16, 10248, "bf16", "normal", 1.0, 1.0, False),
]


@pytest.mark.gpu
@pytest.mark.parametrize("tail", ["default", "fused", "split"])
@pytest.mark.parametrize("B,L,V,dtype,kind,sigma,T,bonus", CASES)
def test_random_cases(B, L, V, dtype, kind, sigma, T, bonus, tail, monkeypatch):
    """The default path (at V <= 1024 one wavefront per sequence) and both
    forms of the general path's tail (one workgroup per sequence, or each
    redraw row spread over several workgroups) against the oracle."""
    if tail != "default":
        monkeypatch.setenv("UNO_VERIFY_SMALL", "0")
        monkeypatch.setenv("UNO_VERIFY_TAIL", tail)
    z, d = verify_inputs(B, L, V, seed=B * 31 + L + V, kind=kind, target_sigma=3.0, draft_sigma=sigma,
                         has_bonus=bonus, dtype=dtype)
    x = _drafts(d, T)
    u = oracle.philox_uniforms(0, 0, 0, B * (L + 1)).reshape(B, L + 1)
    _check(z, d, x, u, T, bonus, dtype, f"B={B} L={L} V={V} {dtype} {kind} sigma={sigma} T={T} bonus={bonus}")


@pytest.mark.gpu
@pytest.mark.parametrize("path", ["default", "general"])
def test_edge_cases_masks_invalid_tokens_broadcast(path, monkeypatch):
    if path == "general":
        monkeypatch.setenv("UNO_VERIFY_SMALL", "0")
    rng = np.random.default_rng(4)
    B, L, V = 6, 5, 300
    z, d = verify_inputs(B, L, V, seed=11, kind="normal", target_sigma=2.0, draft_sigma=1.0, dtype="bf16")
    z[:, :, 200:] = -np.inf            # masked tokens in the target
    d[:, :, :10] = -np.inf             # and in the draft
    x = _drafts(d, 1.0)
    x[1, 2] = V                        # out of range -> sentinel
    x[2, 0] = -5
    x[3, 1] = 250                      # zero target probability -> reject
    u = rng.random((B, L + 1))
    u = np.float32(u).astype(np.float64)
    gpu, ref = _check(z, d, x, u, 1.0, False, "bf16", "masks/invalid tokens")
    assert gpu[0][1] == -1 and gpu[0][2] == -1 and gpu[2][1] == 0
    # stride-0 broadcast of one block to many sequences
    zb, db = z[:1], d[:1]
    xb = np.tile(_drafts(db, 1.0), (50, 1))
    ub = oracle.philox_uniforms(3, 0, 0, 50 * (L + 1)).reshape(50, L + 1)
    _check(zb, db, xb, ub, 1.0, False, "bf16", "broadcast")


@pytest.mark.gpu
@pytest.mark.parametrize("path", ["default", "general"])
def test_q_equal_p_accepts_all_and_disjoint_rejects_first(path, monkeypatch):
    if path == "general":
        monkeypatch.setenv("UNO_VERIFY_SMALL", "0")
    B, L, V = 40, 8, 777
    z, _ = verify_inputs(B, L, V, seed=2, kind="normal", dtype="bf16")
    x = _drafts(z, 0.8)
    u = oracle.philox_uniforms(0, 0, 0, B * (L + 1)).reshape(B, L + 1)
    zt = to_dev(z, "bf16")
    say("verify q == p")
    n_acc, tok, n_emit = uno.block_verify(zt, zt, to_dev(x, "i32"), to_dev(u, "f32"), 0.8, False)
    assert np.all(to_host(n_acc) == L) and np.all(to_host(n_emit) == L)
    np.testing.assert_array_equal(to_host(tok)[:, :L], x)
    # disjoint supports: draft mass on [0, 100), target mass on [100, V)
    zz = np.full((B, L, V), -np.inf, np.float32)
    zz[:, :, 100:] = z[:, :, 100:]
    dd = np.full((B, L, V), -np.inf, np.float32)
    dd[:, :, :100] = z[:, :, :100]
    xd = _drafts(dd, 1.0)
    gpu, _ = _check(zz, dd, xd, u, 1.0, False, "bf16", "disjoint supports")
    assert np.all(gpu[0] == 0) and np.all(gpu[1][:, 0] >= 100)


@pytest.mark.gpu
def test_empty_batch_and_determinism():
    say("verify empty batch")
    e = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    n_acc, tok, n_emit = uno.block_verify(e, e, torch.empty((0, 4), dtype=torch.int32, device="cuda"),
                                          torch.empty((0, 5), dtype=torch.float32, device="cuda"))
    assert n_acc.numel() == 0 and tok.shape == (0, 5)
    B, L, V = 20, 16, 5000
    z, d = verify_inputs(B, L, V, seed=9, dtype="bf16")
    x = _drafts(d, 1.0)
    u = oracle.philox_uniforms(0, 0, 0, B * (L + 1)).reshape(B, L + 1)
    args = (to_dev(z, "bf16"), to_dev(d, "bf16"), to_dev(x, "i32"), to_dev(u, "f32"))
    r1 = [to_host(t) for t in uno.block_verify(*args)]
    r2 = [to_host(t) for t in uno.block_verify(*args)]
    for a, b in zip(r1, r2):
        np.testing.assert_array_equal(a, b)


def _full_vocab_case(B, L, V, kind, sigma, T, seed, check_seqs):
    """GPU-generated full-vocabulary logits; the oracle checks the sampled sequences."""
    say(f"verify full-size B={B} L={L} V={V} {kind} sigma={sigma} T={T}")
    zt, dt = sdev.verify_logits(B, L, V, seed, kind=kind, target_sigma=3.0, draft_sigma=sigma)
    xt = sdev.random_tokens(B, L, V, seed + 1)
    z = to_host(zt[check_seqs]).astype(np.float32)
    d = to_host(dt[check_seqs]).astype(np.float32)
    x_chk = _drafts(d, T, seed=seed)
    xt[torch.as_tensor(check_seqs, device="cuda")] = to_dev(x_chk, "i32")
    u = oracle.philox_uniforms(seed, 0, 0, B * (L + 1)).reshape(B, L + 1)
    n_acc, tok, n_emit = uno.block_verify(zt, dt, xt, to_dev(u, "f32"), T, False)
    torch.cuda.synchronize()
    gpu = tuple(to_host(t)[check_seqs] for t in (n_acc, tok, n_emit))
    uu = u[check_seqs]
    ref = oracle.block_verify(z, d, x_chk, uu, T, False)
    exact, excused, fails = compare_verify(gpu, ref, z, d, uu, T, False)
    print(f"  full-size: exact {exact} excused ties {excused} failures {len(fails)}; "
          f"mean emitted {gpu[2].mean():.2f}", flush=True)
    assert not fails, fails[:5]
    assert excused <= max(1, len(check_seqs) // 50)


@pytest.mark.gpu
def test_layer_b1_full_size():
    wl = WORKLOADS["layer_b1"]
    _full_vocab_case(1, wl.block, wl.vocab, "normal", 1.0, 1.0, wl.seed, np.array([0]))


@pytest.mark.gpu
@pytest.mark.parametrize("sigma", [0.25, 1.0, 4.0])
def test_layer_b64_full_size(sigma):
    wl = WORKLOADS["layer_b64"]
    _full_vocab_case(64, wl.block, wl.vocab, "normal", sigma, 1.0, wl.seed, np.arange(64))


@pytest.mark.gpu
@pytest.mark.parametrize("tail", ["default", "split"])
@pytest.mark.parametrize("T", [0.6, 1.0])
def test_serve_b256_full_size(T, tail, monkeypatch):
    if tail != "default":
        monkeypatch.setenv("UNO_VERIFY_TAIL", tail)
    wl = WORKLOADS["serve_b256"]
    _full_vocab_case(256, wl.block, wl.vocab, "zipf", 0.5, T, wl.seed, np.arange(0, 256, 16))


@pytest.mark.gpu
@pytest.mark.parametrize("tail", ["default", "fused"])
def test_stack32_b32_full_size(tail, monkeypatch):
    if tail != "default":
        monkeypatch.setenv("UNO_VERIFY_TAIL", tail)
    wl = WORKLOADS["stack32_b32"]
    _full_vocab_case(32, wl.block, wl.vocab, "normal", 1.0, 1.0, wl.seed, np.arange(32))


# ---------------------------------------------------------------- early exit
EARLY = [  # B, L, V, dtype, kind, sigma, T, bonus, chunk
    (37, 7, 1000, "bf16", "normal", 1.0, 1.0, False, 3),    # ragged last chunk
    (37, 7, 999, "bf16", "normal", 0.25, 0.6, True, 2),     # bonus row with the last chunk
    (16, 64, 4096, "bf16", "normal", 1.0, 1.0, False, 4),
    (9, 63, 520, "f32", "normal", 4.0, 1.0, True, 16),
    (64, 16, 2048, "bf16", "zipf", 0.5, 0.6, False, 1),     # one position per chunk
    (64, 16, 2048, "bf16", "zipf", 0.5, 0.6, True, 64),     # one chunk: the one-pass schedule
    (300, 2, 17, "f32", "normal", 1.0, 2.0, False, 1),
    (96, 16, 10248, "bf16", "normal", 1.0, 1.0, True, 6),   # one statistics chunk per row, pipelined steps
]


@pytest.mark.gpu
@pytest.mark.parametrize("path", ["default", "general"])
@pytest.mark.parametrize("B,L,V,dtype,kind,sigma,T,bonus,chunk", EARLY)
def test_early_exit_matches_one_pass_and_oracle(B, L, V, dtype, kind, sigma, T, bonus, chunk, path, monkeypatch):
    """Early-exit verification: the same bits as the one-pass verifier, and the oracle's tokens
    (the general path forced at every V, so that its chunk schedule runs on the small vocabularies)."""
    if path == "general":
        monkeypatch.setenv("UNO_VERIFY_SMALL", "0")
    z, d = verify_inputs(B, L, V, seed=B * 37 + L + V, kind=kind, target_sigma=3.0, draft_sigma=sigma,
                         has_bonus=bonus, dtype=dtype)
    x = _drafts(d, T)
    u = oracle.philox_uniforms(0, 0, 0, B * (L + 1)).reshape(B, L + 1)
    args = (to_dev(z, dtype), to_dev(d, dtype), to_dev(x, "i32"), to_dev(u, "f32"), T, bonus)
    say(f"verify early B={B} L={L} V={V} chunk={chunk} bonus={bonus}")
    one = [to_host(t) for t in uno.block_verify(*args)]
    early = [to_host(t) for t in uno.block_verify(*args, early_chunk=chunk)]
    for a, b in zip(one, early):
        np.testing.assert_array_equal(a, b)
    ref = oracle.block_verify(z, d, x, u, T, bonus)
    exact, excused, fails = compare_verify(tuple(early), ref, z, d, u, T, bonus)
    assert not fails, fails[:5]
    assert excused <= max(1, 0.01 * B)


@pytest.mark.gpu
@pytest.mark.parametrize("path", ["default", "general"])
def test_early_exit_invalid_tokens_and_accept_all(path, monkeypatch):
    """Out-of-range tokens past a rejection still give -1; q == p accepts every chunk."""
    if path == "general":
        monkeypatch.setenv("UNO_VERIFY_SMALL", "0")
    B, L, V = 12, 9, 300
    z, d = verify_inputs(B, L, V, seed=5, kind="normal", target_sigma=2.0, draft_sigma=1.0, dtype="bf16")
    x = _drafts(d, 1.0)
    x[1, 8] = V          # invalid token in the last chunk
    x[2, 0] = -1         # invalid token in the first chunk
    u = oracle.philox_uniforms(1, 0, 0, B * (L + 1)).reshape(B, L + 1)
    args = (to_dev(z, "bf16"), to_dev(d, "bf16"), to_dev(x, "i32"), to_dev(u, "f32"), 1.0, False)
    say("verify early: invalid tokens")
    one = [to_host(t) for t in uno.block_verify(*args)]
    early = [to_host(t) for t in uno.block_verify(*args, early_chunk=2)]
    for a, b in zip(one, early):
        np.testing.assert_array_equal(a, b)
    assert early[0][1] == -1 and early[0][2] == -1
    zt = to_dev(z, "bf16")
    xs = _drafts(z, 1.0)
    say("verify early: q == p")
    n_acc, tok, n_emit = uno.block_verify(zt, zt, to_dev(xs, "i32"), to_dev(u, "f32"), 1.0, False, early_chunk=4)
    assert np.all(to_host(n_acc) == L) and np.all(to_host(n_emit) == L)
    np.testing.assert_array_equal(to_host(tok)[:, :L], xs)


@pytest.mark.gpu
def test_early_exit_full_size():
    """Full vocabulary (V = 128256) at 32 x 16 positions: early exit equals one pass."""
    wl = WORKLOADS["stack32_b32"]
    B, L, V = 32, wl.block, wl.vocab
    say(f"verify early full-size B={B} L={L} V={V}")
    zt, dt = sdev.verify_logits(B, L, V, wl.seed, kind="normal", target_sigma=3.0, draft_sigma=1.0)
    d = to_host(dt).astype(np.float32)
    xt = to_dev(_drafts(d, 1.0, seed=wl.seed), "i32")
    u = to_dev(oracle.philox_uniforms(wl.seed, 0, 0, B * (L + 1)).reshape(B, L + 1), "f32")
    one = [to_host(t) for t in uno.block_verify(zt, dt, xt, u, 1.0, False)]
    for chunk in (2, 4):
        early = [to_host(t) for t in uno.block_verify(zt, dt, xt, u, 1.0, False, early_chunk=chunk)]
        for a, b in zip(one, early):
            np.testing.assert_array_equal(a, b)
