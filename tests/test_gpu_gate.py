"""Gate bytes outside {0, 1} on the GPU.

The gate picks a row's pathway: 1 the draft pathway (AR weights plus the
adapter), 0 the verification pathway (AR weights alone) -- "Two Decoupled
Weight Sets" on the aifromscratch.in page.  Any other byte is a caller error
that must not pass silently: the row runs neither pathway, its output row is
NaN, and the row plan counts it (uno_row_plan_gate_errors: count, first row).
Every other row is bitwise the row of the same call with the bad bytes set to
0, and within the bf16 bound of the fp64 oracle on its own gate.
"""

import numpy as np
import pytest
import torch

import lossless_speculative_drafting_amd as uno
import oracle
from gpu_util import say, to_dev, to_host
from parity import BF16_TOL, F32_TOL, floored_rel_err
from synthetic import gemm_inputs


def _bad_gate(M, seed, n_bad):
    rng = np.random.default_rng(seed)
    gate = (rng.random(M) < 0.5).astype(np.uint8)
    bad = np.sort(rng.choice(M, size=n_bad, replace=False))
    gate[bad] = rng.choice([2, 7, 128, 255], size=n_bad)
    return gate, bad


def _check_errors(ge, gate):
    bad = np.nonzero(gate > 1)[0]
    want = [len(bad), int(bad[0]) if len(bad) else -1]
    assert ge.cpu().tolist() == want, (ge.cpu().tolist(), want)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,M,K,N,r,n_bad", [
    ("bf16", 75, 520, 300, 128, 5),     # ragged, several tiles
    ("bf16", 1024, 512, 512, 128, 40),  # many rows, several m tiles of bad rows
    ("bf16", 40, 256, 128, 16, 40),     # every row bad: both segments empty
    ("bf16", 33, 4096, 1024, 128, 1),   # split of K
    ("bf16", 32, 1024, 512, 128, 4),    # 32 rows or fewer: the compact 32-row tile
    ("bf16", 24, 256, 128, 16, 24),     # ... every row bad
    ("f32", 24, 512, 512, 128, 3),      # fp32 correctness path
])
def test_bad_gate_rows_are_nan_and_counted(dtype, M, K, N, r, n_bad):
    gate, bad = _bad_gate(M, M + K + n_bad, n_bad)
    inp = gemm_inputs(M, K, N, r, seed=M + N, dtype=dtype, gate=np.where(gate > 1, 0, gate).astype(np.uint8))
    say("gate bytes outside {0,1}", dtype, M, K, N, r, n_bad)
    args = [to_dev(inp[k], dtype) for k in ("x", "w", "a", "b")]
    ge = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    y = to_host(uno.gated_lora_fwd(*args, to_dev(gate, "u8"), scale=2.0, gate_errors=ge))
    clean = np.where(gate > 1, 0, gate).astype(np.uint8)
    ge0 = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    y0 = to_host(uno.gated_lora_fwd(*args, to_dev(clean, "u8"), scale=2.0, gate_errors=ge0))
    torch.cuda.synchronize()
    _check_errors(ge, gate)
    _check_errors(ge0, clean)
    assert np.all(np.isnan(y[bad])), "rows with an invalid gate byte must be NaN"
    good = gate <= 1
    assert not np.any(np.isnan(y[good]))
    assert np.array_equal(y[good], y0[good]), "valid rows must not depend on the invalid ones"
    if good.any():
        ref = oracle.gated_lora(inp["x"][good], inp["w"], inp["a"], inp["b"], gate[good], 2.0)
        err = floored_rel_err(y[good], ref)
        assert err <= (BF16_TOL if dtype == "bf16" else F32_TOL), err


@pytest.mark.gpu
@pytest.mark.parametrize("tile,split,M", [(None, None, 300), ("256x256w8k64r3", "3", 300), ("64x256b3", None, 300),
                                          (None, None, 30), (None, "1", 30)])
def test_bad_gate_rows_in_grouped_and_swiglu_launches(tile, split, M, monkeypatch):
    """The plan-based launches of a layer: grouped q|k|v-like and SwiGLU gate|up, with the
    planner's tiles, a split of K (reduction launch), the 64 x 256 tile, and at 30 rows the
    compact 32-row tiles (split as planned, or not at all)."""
    if tile:
        monkeypatch.setenv("UNO_GEMM_TILE", tile)
    if split:
        monkeypatch.setenv("UNO_GEMM_SPLIT", split)
    K, r = 1000, 64
    group_n = [256, 128, 128]
    gate, bad = _bad_gate(M, 11, 17)
    clean = np.where(gate > 1, 0, gate).astype(np.uint8)
    say("gate bytes outside {0,1}: grouped and swiglu launches", tile, split)
    parts = [gemm_inputs(M, K, n, r, seed=60 + g, dtype="bf16", gate=clean) for g, n in enumerate(group_n)]
    x = to_dev(parts[0]["x"], "bf16")
    w = torch.cat([to_dev(p["w"], "bf16") for p in parts])
    a = torch.cat([to_dev(p["a"], "bf16") for p in parts])
    b = torch.cat([to_dev(p["b"], "bf16") for p in parts])
    plan, plan0 = uno.RowPlan(to_dev(gate, "u8")), uno.RowPlan(to_dev(clean, "u8"))
    _check_errors(plan.gate_errors(), gate)
    _check_errors(plan0.gate_errors(), clean)
    outs = [to_host(o) for o in uno.gated_gemm_grouped(x, w, uno.lora_down(x, a, plan), b, plan, group_n)]
    outs0 = [to_host(o) for o in uno.gated_gemm_grouped(x, w, uno.lora_down(x, a, plan0), b, plan0, group_n)]
    good = gate <= 1
    for g in range(len(group_n)):
        assert np.all(np.isnan(outs[g][bad])), g
        assert np.array_equal(outs[g][good], outs0[g][good]), g
    # SwiGLU: gate and up projections of 256 columns each
    w_p, b_p = uno.swiglu_pack(w[:256], torch.cat([w[256:], w[256:]])[:256].contiguous(), b[:256],
                               torch.cat([b[256:], b[256:]])[:256].contiguous())
    a2 = torch.cat([a[:r], a[r:2 * r]])
    act = to_host(uno.gated_gemm_swiglu(x, w_p, uno.lora_down(x, a2, plan), b_p, plan))
    act0 = to_host(uno.gated_gemm_swiglu(x, w_p, uno.lora_down(x, a2, plan0), b_p, plan0))
    assert np.all(np.isnan(act[bad]))
    assert np.array_equal(act[good], act0[good])
