"""Gated-LoRA projection on the GPU vs the fp64 oracle.

Small cases run the oracle on every element; the full 8B-layer shapes run the
GPU on the whole batch and the oracle on sampled rows (rows are independent).
bf16 tolerance 2e-2 and fp32 tolerance 1e-4 in the RMS-floored relative error
of tests/parity.py.  Rows with gate 0 must be bitwise equal to the same call
with every gate 0.
"""

import numpy as np
import pytest
import torch

import lossless_speculative_drafting_amd as uno
import oracle
from gpu_util import say, to_dev, to_host
from parity import BF16_TOL, F32_TOL, floored_rel_err
from synthetic import device as sdev
from synthetic import WORKLOADS, gate_vector, gemm_inputs


def _run(inp, dtype, gate=None):
    g = inp["gate"] if gate is None else gate
    y = uno.gated_lora_fwd(to_dev(inp["x"], dtype), to_dev(inp["w"], dtype), to_dev(inp["a"], dtype),
                           to_dev(inp["b"], dtype), to_dev(g, "u8"), scale=2.0)
    torch.cuda.synchronize()
    return to_host(y)


@pytest.mark.gpu
def test_tiny_f32_workload():
    wl = WORKLOADS["tiny"]
    _, K, N = wl.projections[0]
    gate = gate_vector(wl.n_seq, wl.verify_rows, wl.draft_rows)
    inp = gemm_inputs(wl.rows, K, N, 128, wl.seed, "f32", gate=gate)
    say("gemm tiny f32", wl.rows, K, N)
    y = _run(inp, "f32")
    ref = oracle.gated_lora(inp["x"], inp["w"], inp["a"], inp["b"], inp["gate"], 2.0)
    assert floored_rel_err(y, ref) <= F32_TOL
    y0 = _run(inp, "f32", gate=np.zeros_like(gate))
    assert np.array_equal(y[gate == 0], y0[gate == 0])


SMALL = [  # (M, K, N, r, gate pattern)
    (75, 520, 300, 128, "random"),
    (1, 64, 16, 8, "draft"),
    (1, 64, 16, 8, "verify"),
    (33, 4096, 1024, 128, "random"),
    (200, 136, 130, 256, "random"),
    (130, 256, 384, 128, "draft"),
    (130, 256, 384, 128, "verify"),
    (64, 1024, 4096, 128, "seq"),
]


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,N,r,pattern", SMALL)
def test_bf16_small_shapes(M, K, N, r, pattern):
    rng = np.random.default_rng(M * 7 + K + N + r)
    gate = {"random": (rng.random(M) < 0.5).astype(np.uint8), "draft": np.ones(M, np.uint8),
            "verify": np.zeros(M, np.uint8), "seq": gate_vector(M // 32, 16, 16)}[pattern]
    inp = gemm_inputs(M, K, N, r, seed=M + K + N, dtype="bf16", gate=gate)
    say("gemm bf16", M, K, N, r, pattern)
    y = _run(inp, "bf16")
    ref = oracle.gated_lora(inp["x"], inp["w"], inp["a"], inp["b"], gate, 2.0)
    err = floored_rel_err(y, ref)
    assert err <= BF16_TOL, err
    y0 = _run(inp, "bf16", gate=np.zeros_like(gate))
    assert np.array_equal(y[gate == 0], y0[gate == 0]), "verify rows must match the all-verify call bitwise"


@pytest.mark.gpu
def test_empty_batch_is_noop():
    say("gemm empty batch")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((32, 64), dtype=torch.bfloat16, device="cuda")
    a = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((32, 16), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((0,), dtype=torch.uint8, device="cuda")
    assert uno.gated_lora_fwd(x, w, a, b, g).shape == (0, 32)


def _full_shape_case(wl_name, proj):
    wl = WORKLOADS[wl_name]
    shapes = {n: (K, N) for n, K, N in wl.projections}
    K, N = shapes[proj]
    gate = gate_vector(wl.n_seq, wl.verify_rows, wl.draft_rows)
    inp = gemm_inputs(wl.rows, K, N, 128, seed=wl.seed + 17 * [n for n, _, _ in wl.projections].index(proj), dtype="bf16", gate=gate)
    say("gemm full", wl_name, proj, wl.rows, K, N)
    y = _run(inp, "bf16")
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, wl.rows - 1, wl.verify_rows, wl.verify_rows - 1],
                                     rng.choice(wl.rows, size=min(60, wl.rows), replace=False)]))
    ref = oracle.gated_lora(inp["x"][rows], inp["w"], inp["a"], inp["b"], gate[rows], 2.0)
    err = floored_rel_err(y[rows], ref)
    assert err <= BF16_TOL, err


@pytest.mark.gpu
@pytest.mark.parametrize("proj", ["q", "k", "v", "o", "gate", "up", "down"])
def test_layer_b1_projection(proj):
    _full_shape_case("layer_b1", proj)


@pytest.mark.gpu
@pytest.mark.parametrize("proj", ["q", "k", "down"])
def test_layer_b64_projection(proj):
    _full_shape_case("layer_b64", proj)


@pytest.mark.gpu
@pytest.mark.parametrize("proj", ["up", "down"])
def test_serve_b256_projection(proj):
    _full_shape_case("serve_b256", proj)


@pytest.mark.gpu
def test_deterministic_repeat():
    inp = gemm_inputs(300, 1024, 512, 128, seed=3, dtype="bf16")
    say("gemm determinism")
    assert np.array_equal(_run(inp, "bf16"), _run(inp, "bf16"))


@pytest.mark.gpu
@pytest.mark.parametrize("tile", ["64x128", "128x128", "128x128b3", "128x128b4", "128x128b5", "128x128b4kg2", "128x256",
                                  "256x128", "256x128k64b3kg2", "256x256", "256x192w8k64r3",
                                  "256x256k64", "256x256k64r3", "256x256w8", "256x256w8k64", "256x256w8k64r3",
                                  "256x256pp", "128x192b3", "128x192b4", "128x192b3kg2", "128x192b4kg2",
                                  "64x256", "64x256b3"])
def test_every_tile_shape_ragged(tile, monkeypatch):
    """Each workgroup tile on a problem ragged in M, N and K, through the split steps."""
    monkeypatch.setenv("UNO_GEMM_TILE", tile)
    M, K, N, r = 300, 1000, 700, 128
    rng = np.random.default_rng(11)
    gate = (rng.random(M) < 0.4).astype(np.uint8)
    inp = gemm_inputs(M, K, N, r, seed=21, dtype="bf16", gate=gate)
    say("gemm tile", tile)
    x, w = to_dev(inp["x"], "bf16"), to_dev(inp["w"], "bf16")
    a, b = to_dev(inp["a"], "bf16"), to_dev(inp["b"], "bf16")
    plan = uno.RowPlan(to_dev(gate, "u8"))
    t = uno.lora_down(x, a, plan, 2.0)
    y = to_host(uno.gated_gemm(x, w, t, b, plan))
    ref = oracle.gated_lora(inp["x"], inp["w"], inp["a"], inp["b"], gate, 2.0)
    err = floored_rel_err(y, ref)
    assert err <= BF16_TOL, err
    y_full = _run(inp, "bf16")
    assert np.array_equal(y, y_full), "split steps and the one-call projection must agree bitwise"


@pytest.mark.gpu
@pytest.mark.parametrize("tile,split", [("128x192b4kg2", 3), ("128x192b3", 2), ("128x128b4kg2", 4)])
def test_tiles_with_split_k_ragged(tile, split, monkeypatch):
    """A tile with K split over workgroups (fp32 partials, ordered reduction) on a ragged problem."""
    monkeypatch.setenv("UNO_GEMM_TILE", tile)
    monkeypatch.setenv("UNO_GEMM_SPLIT", str(split))
    M, K, N, r = 300, 1000, 700, 128
    rng = np.random.default_rng(12)
    gate = (rng.random(M) < 0.4).astype(np.uint8)
    inp = gemm_inputs(M, K, N, r, seed=22, dtype="bf16", gate=gate)
    say("gemm tile split", tile, split)
    x, w = to_dev(inp["x"], "bf16"), to_dev(inp["w"], "bf16")
    a, b = to_dev(inp["a"], "bf16"), to_dev(inp["b"], "bf16")
    plan = uno.RowPlan(to_dev(gate, "u8"))
    t = uno.lora_down(x, a, plan, 2.0)
    y = to_host(uno.gated_gemm(x, w, t, b, plan))
    ref = oracle.gated_lora(inp["x"], inp["w"], inp["a"], inp["b"], gate, 2.0)
    err = floored_rel_err(y, ref)
    assert err <= BF16_TOL, err


@pytest.mark.gpu
@pytest.mark.parametrize("t_tile", ["64b2", "128", "64kg2"])
def test_lora_down_tiles_agree(t_tile, monkeypatch):
    """The LoRA down-projection gives the same T bits with every one-group tile and
    buffer count (each output sums the same K slices in the same order).  Two K
    groups sum the even and the odd K sub-steps apart and add the two sums, so
    there T agrees to bf16 rounding instead."""
    M, K, r = 300, 2048, 128  # K = 2048: four K splits for every tile
    rng = np.random.default_rng(12)
    gate = (rng.random(M) < 0.5).astype(np.uint8)
    inp = gemm_inputs(M, K, 256, r, seed=22, dtype="bf16", gate=gate)
    say("lora_down tile", t_tile)
    x, a = to_dev(inp["x"], "bf16"), to_dev(inp["a"], "bf16")
    plan = uno.RowPlan(to_dev(gate, "u8"))
    t_default = uno.lora_down(x, a, plan, 2.0).clone()
    monkeypatch.setenv("UNO_T_TILE", t_tile)
    t_forced = uno.lora_down(x, a, plan, 2.0)
    if "kg2" in t_tile:
        err = floored_rel_err(to_host(t_forced).astype(np.float64), to_host(t_default).astype(np.float64))
        assert err <= BF16_TOL, err
    else:
        assert torch.equal(t_default, t_forced)


EPILOGUE = [  # M, K, N (per projection), forced tile or None, forced split or None
    (1024, 512, 512, None, None),       # planner's tiles, one K pass
    (300, 1000, 512, "256x256w8", "2"),  # ragged M and K, split-K: the reduction applies the epilogue
    (32, 256, 256, None, None),          # few rows: the 128 x 256 tile (SwiGLU) / 64 x 128 (residual)
    (96, 512, 768, "128x256", None),
    (300, 1000, 512, "256x256w8k64r3", None),  # split ring, ragged
    (32, 1000, 768, "64x256b3", "3"),     # few rows, the weight-streaming tile, ragged K, split-K
    (60, 512, 512, "64x256", None),       # two stage buffers, ragged M
]


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,N,tile,split", EPILOGUE)
def test_residual_epilogue_is_separate_add(M, K, N, tile, split, monkeypatch):
    """uno_gated_gemm_residual == uno_residual_add(y, uno_gated_gemm(...)), bit for bit."""
    if tile:
        monkeypatch.setenv("UNO_GEMM_TILE", tile)
    if split:
        monkeypatch.setenv("UNO_GEMM_SPLIT", split)
    rng = np.random.default_rng(M + N)
    gate = (rng.random(M) < 0.5).astype(np.uint8)
    inp = gemm_inputs(M, K, N, 128, seed=M + K, dtype="bf16", gate=gate)
    say("residual epilogue", M, K, N, tile, split)
    x, w = to_dev(inp["x"], "bf16"), to_dev(inp["w"], "bf16")
    a, b = to_dev(inp["a"], "bf16"), to_dev(inp["b"], "bf16")
    plan = uno.RowPlan(to_dev(gate, "u8"))
    t = uno.lora_down(x, a, plan, 2.0)
    y0 = sdev.randn((M, N), 2.0, M + 5)
    ref = uno.residual_add(y0, uno.gated_gemm(x, w, t, b, plan))
    y = y0.clone()
    uno.gated_gemm_residual(x, w, t, b, plan, y)
    assert torch.equal(y, ref)


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,N,tile,split", EPILOGUE)
def test_swiglu_epilogue_is_separate_silu_mul(M, K, N, tile, split, monkeypatch):
    """uno_gated_gemm_swiglu on packed weights == silu_mul of the gate and up projections, bit for
    bit (same tile family and split), and within the bf16 bound of the fp64 oracle."""
    # the same tile family and K split on both sides (the two plans may
    # otherwise differ, and K-group tiles sum alternate sub-steps apart)
    monkeypatch.setenv("UNO_GEMM_TILE", tile or "256x256w8k64r3")
    monkeypatch.setenv("UNO_GEMM_SPLIT", split or "1")
    rng = np.random.default_rng(M + 3 * N)
    gate = (rng.random(M) < 0.5).astype(np.uint8)
    g_in = gemm_inputs(M, K, N, 128, seed=M + 1, dtype="bf16", gate=gate)
    u_in = gemm_inputs(M, K, N, 128, seed=M + 2, dtype="bf16", gate=gate)
    say("swiglu epilogue", M, K, N, tile, split)
    x = to_dev(g_in["x"], "bf16")
    wg, wu = to_dev(g_in["w"], "bf16"), to_dev(u_in["w"], "bf16")
    ag, au = to_dev(g_in["a"], "bf16"), to_dev(u_in["a"], "bf16")
    bg, bu = to_dev(g_in["b"], "bf16"), to_dev(u_in["b"], "bf16")
    plan = uno.RowPlan(to_dev(gate, "u8"))
    t = uno.lora_down(x, torch.cat([ag, au], 0), plan, 2.0)       # [T_gate | T_up]
    w_p, b_p = uno.swiglu_pack(wg, wu, bg, bu)
    act = uno.gated_gemm_swiglu(x, w_p, t, b_p, plan)
    g, u = uno.gated_gemm_grouped(x, torch.cat([wg, wu], 0), t, torch.cat([bg, bu], 0), plan, [N, N])
    assert torch.equal(act, uno.silu_mul(g, u))
    g_ref = oracle.gated_lora(g_in["x"], g_in["w"], g_in["a"], g_in["b"], gate, 2.0)
    u_ref = oracle.gated_lora(g_in["x"], u_in["w"], u_in["a"], u_in["b"], gate, 2.0)
    gh, uh, ah = to_host(g), to_host(u), to_host(act)
    # each projection within the bf16 bound, and the epilogue within it of the
    # fp64 silu(g) u of the GPU's own bf16 g and u
    assert floored_rel_err(gh, g_ref) <= BF16_TOL and floored_rel_err(uh, u_ref) <= BF16_TOL
    assert floored_rel_err(ah, oracle.stack.silu_mul(gh, uh)) <= BF16_TOL
    # against silu(g) u of the exact projections the two projections' relative
    # errors add (an error in g is multiplied by |u|, which the row-RMS floor
    # of the product does not scale with): twice the bound
    err = floored_rel_err(ah, oracle.stack.silu_mul(g_ref, u_ref))
    print(f"  floored rel err vs exact {err:.3e}", flush=True)
    assert err <= 2 * BF16_TOL, err


@pytest.mark.gpu
@pytest.mark.parametrize("M", [1, 17, 32])
def test_swiglu_default_plan_few_rows(M, monkeypatch):
    """The SwiGLU launch as planned for a single sequence (32 rows or fewer: the compact
    32 x 256 tile) against the oracle's silu(g) u of the exact projections."""
    for var in ("UNO_GEMM_TILE", "UNO_GEMM_SPLIT", "UNO_STREAM"):
        monkeypatch.delenv(var, raising=False)
    K, N = 1024, 512
    rng = np.random.default_rng(M + 77)
    gate = (rng.random(M) < 0.5).astype(np.uint8)
    g_in = gemm_inputs(M, K, N, 128, seed=M + 11, dtype="bf16", gate=gate)
    u_in = gemm_inputs(M, K, N, 128, seed=M + 12, dtype="bf16", gate=gate)
    say("swiglu default plan", M, K, N)
    x = to_dev(g_in["x"], "bf16")
    plan = uno.RowPlan(to_dev(gate, "u8"))
    t = uno.lora_down(x, torch.cat([to_dev(g_in["a"], "bf16"), to_dev(u_in["a"], "bf16")], 0), plan, 2.0)
    w_p, b_p = uno.swiglu_pack(to_dev(g_in["w"], "bf16"), to_dev(u_in["w"], "bf16"), to_dev(g_in["b"], "bf16"),
                               to_dev(u_in["b"], "bf16"))
    act = to_host(uno.gated_gemm_swiglu(x, w_p, t, b_p, plan))
    g_ref = oracle.gated_lora(g_in["x"], g_in["w"], g_in["a"], g_in["b"], gate, 2.0)
    u_ref = oracle.gated_lora(g_in["x"], u_in["w"], u_in["a"], u_in["b"], gate, 2.0)
    err = floored_rel_err(act, oracle.stack.silu_mul(g_ref, u_ref))
    print(f"  floored rel err vs exact {err:.3e}", flush=True)
    assert err <= 2 * BF16_TOL, err


@pytest.mark.gpu
@pytest.mark.parametrize("M", [1, 20, 32])
def test_swiglu_compact_tile_pairs_half_blocks(M, monkeypatch):
    """The compact SwiGLU tile (32 rows x 128 columns: half a gate block and the same half
    of its up block) against the 64 x 256 tile it replaces, both with one K pass and one
    K group: the same K slices in the same order, so the same bits; with K split three
    ways (partials in weight-row order, summed by the reduction) within the bf16 bound."""
    K, N_half, r = 1024, 768, 128
    rng = np.random.default_rng(M + 91)
    gate = (rng.random(M) < 0.5).astype(np.uint8)
    g_in = gemm_inputs(M, K, N_half, r, seed=M + 21, dtype="bf16", gate=gate)
    u_in = gemm_inputs(M, K, N_half, r, seed=M + 22, dtype="bf16", gate=gate)
    say("swiglu compact tile", M)
    for var in ("UNO_GEMM_TILE", "UNO_GEMM_SPLIT", "UNO_STREAM", "UNO_COMPACT"):
        monkeypatch.delenv(var, raising=False)
    x = to_dev(g_in["x"], "bf16")
    plan = uno.RowPlan(to_dev(gate, "u8"))
    t = uno.lora_down(x, torch.cat([to_dev(g_in["a"], "bf16"), to_dev(u_in["a"], "bf16")], 0), plan, 2.0)
    w_p, b_p = uno.swiglu_pack(to_dev(g_in["w"], "bf16"), to_dev(u_in["w"], "bf16"), to_dev(g_in["b"], "bf16"),
                               to_dev(u_in["b"], "bf16"))
    monkeypatch.setenv("UNO_GEMM_SPLIT", "1")
    act_c = to_host(uno.gated_gemm_swiglu(x, w_p, t, b_p, plan))
    monkeypatch.setenv("UNO_COMPACT", "0")
    act_64 = to_host(uno.gated_gemm_swiglu(x, w_p, t, b_p, plan))
    assert np.array_equal(act_c, act_64)
    monkeypatch.delenv("UNO_COMPACT")
    monkeypatch.setenv("UNO_GEMM_SPLIT", "3")
    act_s = to_host(uno.gated_gemm_swiglu(x, w_p, t, b_p, plan))
    assert floored_rel_err(act_s.astype(np.float64), act_c.astype(np.float64)) <= BF16_TOL
    g_ref = oracle.gated_lora(g_in["x"], g_in["w"], g_in["a"], g_in["b"], gate, 2.0)
    u_ref = oracle.gated_lora(g_in["x"], u_in["w"], u_in["a"], u_in["b"], gate, 2.0)
    err = floored_rel_err(act_c, oracle.stack.silu_mul(g_ref, u_ref))
    assert err <= 2 * BF16_TOL, err


@pytest.mark.gpu
def test_swiglu_pack_layout():
    """Packed rows and the block-diagonal B, checked element by element on the host."""
    N, K, r = 256, 64, 16
    rng = np.random.default_rng(8)
    mats = [rng.standard_normal(s).astype(np.float32) for s in ((N, K), (N, K), (N, r), (N, r))]
    w_p, b_p = (to_host(t) for t in uno.swiglu_pack(*(to_dev(m, "bf16") for m in mats)))
    wg, wu, bg, bu = (to_host(to_dev(m, "bf16")) for m in mats)
    for R in range(2 * N):
        src = (R // 256) * 128 + R % 128
        up = R % 256 >= 128
        np.testing.assert_array_equal(w_p[R], (wu if up else wg)[src])
        want = np.zeros(2 * r, np.float32)
        if up:
            want[r:] = bu[src]
        else:
            want[:r] = bg[src]
        np.testing.assert_array_equal(b_p[R], want)


GROUPED = [  # (M, K, group sizes, r)
    (75, 256, (256, 128, 72), 64),          # ragged M and last group; K = 256 never splits
    (300, 1000, (384, 256), 128),           # ragged K
    (64, 4096, (4096, 1024, 1024), 128),    # q | k | v of the 8B layer, 2 x [16 | 16] rows
    (96, 512, (128, 128, 128, 128), 16),    # four groups
    (32, 4096, (4096, 1024, 1024), 128),    # q | k | v of one sequence: the compact 32-row tile
    (29, 1000, (256, 128, 72), 64),         # compact tile, ragged K and last group
]


def _group_inputs(M, K, group_n, r, seed, gate):
    parts = [gemm_inputs(M, K, n, r, seed=seed + g, dtype="bf16", gate=gate) for g, n in enumerate(group_n)]
    x = parts[0]["x"]
    return x, [(p["w"], p["a"], p["b"]) for p in parts]


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,group_n,r", GROUPED)
def test_grouped_gemm_vs_oracle(M, K, group_n, r):
    _grouped_case(M, K, group_n, r)


@pytest.mark.gpu
@pytest.mark.parametrize("tile,M,K,group_n,r", [
    ("128x192b4kg2", 64, 4096, (4096, 1024, 1024), 128),  # q | k | v: tiles across 4096 and 5120
    ("128x192b3", 96, 512, (128, 128, 128, 128), 16),     # tiles over two groups; r not a stage multiple
    ("256x256w8k64r3", 96, 512, (128, 128, 128, 128), 64),  # split ring, two groups per tile
    ("128x128b4kg2", 75, 1000, (256, 128, 72), 64),       # group ends on tile edges (no straddle)
])
def test_grouped_gemm_tiles_across_groups(tile, M, K, group_n, r, monkeypatch):
    """Tiles whose columns fall in several output groups: each group's columns
    take their own slice of T (the other slices read zero B rows)."""
    monkeypatch.setenv("UNO_GEMM_TILE", tile)
    _grouped_case(M, K, group_n, r, check_single=False)


def _grouped_case(M, K, group_n, r, check_single=True):
    rng = np.random.default_rng(M + K)
    gate = (rng.random(M) < 0.5).astype(np.uint8)
    x, groups = _group_inputs(M, K, group_n, r, 40 + M, gate)
    say("gemm grouped", M, K, group_n, r)
    xd = to_dev(x, "bf16")
    w = torch.cat([to_dev(g[0], "bf16") for g in groups])
    a = torch.cat([to_dev(g[1], "bf16") for g in groups])
    b = torch.cat([to_dev(g[2], "bf16") for g in groups])
    plan = uno.RowPlan(to_dev(gate, "u8"))
    t = uno.lora_down(xd, a, plan, 2.0)
    outs = [to_host(o) for o in uno.gated_gemm_grouped(xd, w, t, b, plan, group_n)]
    for g, (wg, ag, bg) in enumerate(groups):
        ref = oracle.gated_lora(x, wg, ag, bg, gate, 2.0)
        err = floored_rel_err(outs[g], ref)
        assert err <= BF16_TOL, (g, err)
    # verify rows are those of the same grouped call with every gate 0
    plan0 = uno.RowPlan(to_dev(np.zeros_like(gate), "u8"))
    t0 = uno.lora_down(xd, a, plan0, 2.0)
    outs0 = [to_host(o) for o in uno.gated_gemm_grouped(xd, w, t0, b, plan0, group_n)]
    for g in range(len(group_n)):
        assert np.array_equal(outs[g][gate == 0], outs0[g][gate == 0])
    if K == 256 and check_single:
        # no split anywhere: each group equals its own ungrouped call bitwise
        for g, (wg, ag, bg) in enumerate(groups):
            tg = uno.lora_down(xd, to_dev(ag, "bf16"), plan, 2.0)
            yg = to_host(uno.gated_gemm(xd, to_dev(wg, "bf16"), tg, to_dev(bg, "bf16"), plan))
            assert np.array_equal(yg, outs[g]), g


STREAM = [  # M, K, N, r, gate pattern: 32 rows or fewer run the weight-streaming kernel
    (1, 64, 16, 8, "draft"),
    (7, 1000, 300, 16, "random"),      # ragged K (a partial last chunk) and N
    (20, 520, 1024, 128, "random"),
    (32, 4096, 1024, 128, "seq"),      # one sequence of [16 verify | 16 draft]
    (32, 4096, 700, 128, "verify"),
    (32, 2048, 96, 256, "draft"),
    (29, 14336, 256, 128, "random"),   # the down-projection's depth
]


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,N,r,pattern", STREAM)
def test_weight_streaming_kernel(M, K, N, r, pattern, monkeypatch):
    """The weight-streaming kernel (forced for the plain epilogue; its LoRA down-projection is
    split over K) against the oracle; verify rows bitwise those of an all-verify call; the
    split steps equal the one call."""
    monkeypatch.setenv("UNO_GEMM_TILE", "stream")
    rng = np.random.default_rng(M * 3 + K + N)
    gate = {"random": (rng.random(M) < 0.5).astype(np.uint8), "draft": np.ones(M, np.uint8),
            "verify": np.zeros(M, np.uint8), "seq": gate_vector(1, M // 2, M - M // 2)}[pattern]
    inp = gemm_inputs(M, K, N, r, seed=M + 2 * K + N, dtype="bf16", gate=gate)
    say("gemm streaming", M, K, N, r, pattern)
    y = _run(inp, "bf16")
    ref = oracle.gated_lora(inp["x"], inp["w"], inp["a"], inp["b"], gate, 2.0)
    err = floored_rel_err(y, ref)
    assert err <= BF16_TOL, err
    y0 = _run(inp, "bf16", gate=np.zeros_like(gate))
    assert np.array_equal(y[gate == 0], y0[gate == 0]), "verify rows must match the all-verify call bitwise"
    x, w = to_dev(inp["x"], "bf16"), to_dev(inp["w"], "bf16")
    a, b = to_dev(inp["a"], "bf16"), to_dev(inp["b"], "bf16")
    plan = uno.RowPlan(to_dev(gate, "u8"))
    t = uno.lora_down(x, a, plan, 2.0)
    assert np.array_equal(to_host(uno.gated_gemm(x, w, t, b, plan)), y)


COMPACT = [  # M, K, N, r, gate pattern, forced tile (None: the planner's), forced split (None: planned)
    (1, 64, 16, 8, "draft", None, None),
    (1, 64, 16, 8, "verify", None, None),
    (7, 1000, 300, 16, "random", "32x128b4kg2", None),    # ragged K (a partial last stage) and N
    (20, 520, 1024, 128, "random", "32x128b7kg2", "3"),
    (32, 4096, 1024, 128, "seq", None, None),             # one sequence of [16 verify | 16 draft]
    (32, 4096, 700, 128, "verify", None, None),
    (32, 2048, 96, 256, "draft", "32x128b7kg2", "1"),     # r = 256: four extension stages, no split
    (29, 14336, 256, 128, "random", None, None),          # the down-projection's depth
    (31, 1000, 512, 64, "random", "32x256b4", "2"),       # a 256-column compact tile on a plain epilogue
    (30, 1000, 640, 64, "random", "32x128w2b7", None),    # the SwiGLU form (one K group) on a plain epilogue
]


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,N,r,pattern,tile,split", COMPACT)
def test_compact_tiles(M, K, N, r, pattern, tile, split, monkeypatch):
    """The 32-row tiles (rows of both segments compacted into one band) against the oracle;
    verify rows bitwise those of an all-verify call; the split steps equal the one call."""
    for var, val in (("UNO_GEMM_TILE", tile), ("UNO_GEMM_SPLIT", split)):
        if val is None:
            monkeypatch.delenv(var, raising=False)
        else:
            monkeypatch.setenv(var, val)
    monkeypatch.delenv("UNO_COMPACT", raising=False)
    rng = np.random.default_rng(M * 5 + K + N)
    gate = {"random": (rng.random(M) < 0.5).astype(np.uint8), "draft": np.ones(M, np.uint8),
            "verify": np.zeros(M, np.uint8), "seq": gate_vector(1, M // 2, M - M // 2)}[pattern]
    inp = gemm_inputs(M, K, N, r, seed=M + 3 * K + N, dtype="bf16", gate=gate)
    say("gemm compact", M, K, N, r, pattern, tile, split)
    y = _run(inp, "bf16")
    ref = oracle.gated_lora(inp["x"], inp["w"], inp["a"], inp["b"], gate, 2.0)
    err = floored_rel_err(y, ref)
    assert err <= BF16_TOL, err
    y0 = _run(inp, "bf16", gate=np.zeros_like(gate))
    assert np.array_equal(y[gate == 0], y0[gate == 0]), "verify rows must match the all-verify call bitwise"
    x, w = to_dev(inp["x"], "bf16"), to_dev(inp["w"], "bf16")
    a, b = to_dev(inp["a"], "bf16"), to_dev(inp["b"], "bf16")
    plan = uno.RowPlan(to_dev(gate, "u8"))
    t = uno.lora_down(x, a, plan, 2.0)
    assert np.array_equal(to_host(uno.gated_gemm(x, w, t, b, plan)), y)


@pytest.mark.gpu
@pytest.mark.parametrize("M", [1, 16, 32])
def test_compact_tiles_match_64_row_tiles(M, monkeypatch):
    """The compact tile against the 64-row tile it replaces at few rows (UNO_COMPACT=0), on a
    batch-1 q projection: the same sums up to the fp32 order of the split (bf16 bound), and
    with one K split and one K group each, the same bits."""
    K, N, r = 4096, 1024, 128
    rng = np.random.default_rng(M + 3)
    gate = (rng.random(M) < 0.5).astype(np.uint8)
    inp = gemm_inputs(M, K, N, r, seed=M + 9, dtype="bf16", gate=gate)
    say("gemm compact vs 64-row", M)
    for var in ("UNO_GEMM_TILE", "UNO_GEMM_SPLIT", "UNO_STREAM"):
        monkeypatch.delenv(var, raising=False)
    y_c = _run(inp, "bf16")
    monkeypatch.setenv("UNO_COMPACT", "0")
    y_p = _run(inp, "bf16")
    assert floored_rel_err(y_c.astype(np.float64), y_p.astype(np.float64)) <= BF16_TOL
    monkeypatch.setenv("UNO_GEMM_SPLIT", "1")
    monkeypatch.setenv("UNO_GEMM_TILE", "64x128")
    y_p1 = _run(inp, "bf16")
    monkeypatch.setenv("UNO_GEMM_TILE", "32x256b4")
    y_c1 = _run(inp, "bf16")
    assert np.array_equal(y_c1, y_p1), "one K pass, one K group: same K slices in the same order"


@pytest.mark.gpu
@pytest.mark.parametrize("t_split", ["1", "3", "16"])
def test_weight_streaming_lora_down_splits_agree(t_split, monkeypatch):
    """T from the streaming down-projection: the oracle's scale (x A) within bf16 rounding
    for every split of K (fp32 partials summed in split order)."""
    M, K, r = 30, 4096, 384
    rng = np.random.default_rng(40)
    gate = (rng.random(M) < 0.5).astype(np.uint8)
    inp = gemm_inputs(M, K, 64, r, seed=41, dtype="bf16", gate=gate)
    monkeypatch.setenv("UNO_T_SPLIT", t_split)
    say("streaming lora_down split", t_split)
    x, a = to_dev(inp["x"], "bf16"), to_dev(inp["a"], "bf16")
    plan = uno.RowPlan(to_dev(gate, "u8"))
    t = to_host(uno.lora_down(x, a, plan, 2.0)).reshape(-1, r)
    Md = int(gate.sum())
    ref = 2.0 * inp["x"][gate == 1].astype(np.float64) @ inp["a"].astype(np.float64).T
    assert floored_rel_err(t[:Md], ref) <= BF16_TOL
    assert np.all(t[Md:(Md + 31) // 32 * 32] == 0), "padding rows of T are zero"


@pytest.mark.gpu
@pytest.mark.parametrize("M", [1, 17, 32])
def test_weight_streaming_grouped_swiglu_residual(M, monkeypatch):
    """The streaming kernel's epilogues on a layer's shapes (forced for every launch):
    grouped q|k|v against the oracle per group, SwiGLU bitwise silu_mul of the grouped
    gate|up, residual add bitwise the separate add."""
    monkeypatch.setenv("UNO_GEMM_TILE", "stream")
    K, r = 512, 128
    rng = np.random.default_rng(M + 5)
    gate = (rng.random(M) < 0.5).astype(np.uint8)
    group_n = (512, 128, 128)
    x, groups = _group_inputs(M, K, group_n, r, 90 + M, gate)
    say("streaming epilogues", M)
    xd = to_dev(x, "bf16")
    w = torch.cat([to_dev(g[0], "bf16") for g in groups])
    a = torch.cat([to_dev(g[1], "bf16") for g in groups])
    b = torch.cat([to_dev(g[2], "bf16") for g in groups])
    plan = uno.RowPlan(to_dev(gate, "u8"))
    t = uno.lora_down(xd, a, plan, 2.0)
    outs = [to_host(o) for o in uno.gated_gemm_grouped(xd, w, t, b, plan, list(group_n))]
    for g, (wg, ag, bg) in enumerate(groups):
        err = floored_rel_err(outs[g], oracle.gated_lora(x, wg, ag, bg, gate, 2.0))
        assert err <= BF16_TOL, (g, err)
    # SwiGLU over the first two groups as gate (512) and up (2 x 128 -> 256 rows repeated)
    wg, wu = w[:256].contiguous(), w[256:512].contiguous()
    bg, bu = b[:256].contiguous(), b[256:512].contiguous()
    t2 = uno.lora_down(xd, torch.cat([a[:r], a[r:2 * r]]), plan, 2.0)
    w_p, b_p = uno.swiglu_pack(wg, wu, bg, bu)
    act = uno.gated_gemm_swiglu(xd, w_p, t2, b_p, plan)
    gg, uu = uno.gated_gemm_grouped(xd, torch.cat([wg, wu]), t2, torch.cat([bg, bu]), plan, [256, 256])
    assert torch.equal(act, uno.silu_mul(gg, uu))
    y0 = sdev.randn((M, 256), 2.0, M + 9)
    ref = uno.residual_add(y0, uno.gated_gemm(xd, wg, uno.lora_down(xd, a[:r].contiguous(), plan, 2.0), bg, plan))
    y = y0.clone()
    uno.gated_gemm_residual(xd, wg, uno.lora_down(xd, a[:r].contiguous(), plan, 2.0), bg, plan, y)
    assert torch.equal(y, ref)


def _sampled_rows(M, gate, extra=48, seed=6):
    rng = np.random.default_rng(seed)
    first_draft = int(np.argmax(gate == 1)) if gate.any() else 0
    return np.unique(np.concatenate([[0, M - 1, first_draft, max(first_draft - 1, 0)],
                                     rng.choice(M, size=min(extra, M), replace=False)]))


@pytest.mark.gpu
def test_layer_b64_grouped_qkv_launch():
    """The batch-64 layer's grouped q|k|v launch (M = 2048, N = 4096 + 1024 + 1024, the
    planner's tile) against the oracle on sampled rows, per group, at the bf16 bound."""
    wl = WORKLOADS["layer_b64"]
    gate = gate_vector(wl.n_seq, wl.verify_rows, wl.draft_rows)
    M, K, r = wl.rows, 4096, 128
    group_n = [4096, 1024, 1024]
    say("layer_b64 grouped q|k|v", M)
    ws = [sdev.projection_weights(K, n, 5000 + 10 * g) for g, n in enumerate(group_n)]
    x = sdev.randn((M, K), 1.0, 5101)
    w = torch.cat([p[0] for p in ws])
    a = torch.cat([p[1] for p in ws])
    b = torch.cat([p[2] for p in ws])
    plan = uno.RowPlan(to_dev(gate, "u8"))
    t = uno.lora_down(x, a, plan, 2.0)
    outs = uno.gated_gemm_grouped(x, w, t, b, plan, group_n)
    rows = _sampled_rows(M, gate)
    xh = to_host(x)[rows]
    for g, (wg, ag, bg) in enumerate(ws):
        ref = oracle.gated_lora(xh, to_host(wg), to_host(ag), to_host(bg), gate[rows], 2.0)
        err = floored_rel_err(to_host(outs[g])[rows], ref)
        print(f"  group {g}: floored rel err {err:.3e}", flush=True)
        assert err <= BF16_TOL, (g, err)


@pytest.mark.gpu
def test_layer_b64_swiglu_launch(monkeypatch):
    """The batch-64 layer's SwiGLU gate|up launch (M = 2048, N_half = 14336, r = 2 x 128)
    against the oracle at the bf16 bound, stage by stage: the gate and up projections (the
    grouped launch with the same tile) against the oracle on sampled rows; the fused launch
    bitwise silu_mul of those; and the fused output against the fp64 silu(g) u of the GPU's
    own bf16 g and u.  (Against silu(g) u of the exact projections the error is the sum of
    the two projections' and is reported, not bounded here: an error in g is multiplied
    by |u|.)"""
    monkeypatch.setenv("UNO_GEMM_TILE", "256x256w8k64r3")  # a planner candidate at this size
    monkeypatch.setenv("UNO_GEMM_SPLIT", "1")
    wl = WORKLOADS["layer_b64"]
    gate = gate_vector(wl.n_seq, wl.verify_rows, wl.draft_rows)
    M, K, Nh, r = wl.rows, 4096, 14336, 128
    say("layer_b64 swiglu gate|up", M)
    wg, ag, bg = sdev.projection_weights(K, Nh, 6000)
    wu, au, bu = sdev.projection_weights(K, Nh, 6010)
    x = sdev.randn((M, K), 1.0, 6101)
    plan = uno.RowPlan(to_dev(gate, "u8"))
    t = uno.lora_down(x, torch.cat([ag, au]), plan, 2.0)
    w_p, b_p = uno.swiglu_pack(wg, wu, bg, bu)
    act = uno.gated_gemm_swiglu(x, w_p, t, b_p, plan)
    g, u = uno.gated_gemm_grouped(x, torch.cat([wg, wu]), t, torch.cat([bg, bu]), plan, [Nh, Nh])
    assert torch.equal(act, uno.silu_mul(g, u))
    rows = _sampled_rows(M, gate)
    xh = to_host(x)[rows]
    g_ref = oracle.gated_lora(xh, to_host(wg), to_host(ag), to_host(bg), gate[rows], 2.0)
    u_ref = oracle.gated_lora(xh, to_host(wu), to_host(au), to_host(bu), gate[rows], 2.0)
    gh, uh, ah = to_host(g)[rows], to_host(u)[rows], to_host(act)[rows]
    errs = {"gate": floored_rel_err(gh, g_ref), "up": floored_rel_err(uh, u_ref),
            "act vs silu(g_gpu) u_gpu": floored_rel_err(ah, oracle.stack.silu_mul(gh, uh)),
            "act vs exact": floored_rel_err(ah, oracle.stack.silu_mul(g_ref, u_ref))}
    print("  " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()), flush=True)
    assert errs["gate"] <= BF16_TOL and errs["up"] <= BF16_TOL
    assert errs["act vs silu(g_gpu) u_gpu"] <= BF16_TOL
    assert errs["act vs exact"] <= 2 * BF16_TOL
