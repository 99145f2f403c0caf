"""Layer-stack glue and the layer stack on the GPU vs the oracle.

Glue kernels are compared elementwise with the fp64 oracle (bf16 output
rounding bounds the error by 2^-8 relative; the test uses 1e-2 floored).
Projections inside the stack are checked with teacher forcing: each
projection's recorded bf16 input goes through the oracle and is compared with
the projection's output at the 2e-2 bound.
"""

import numpy as np
import pytest
import torch

import lossless_speculative_drafting_amd as uno
import oracle
from gpu_util import say, to_dev, to_host
from parity import BF16_TOL, floored_rel_err
from synthetic import WORKLOADS, bf16_round, gate_vector
from synthetic import device as sdev
from lossless_speculative_drafting_amd.stack import PROJECTIONS


@pytest.mark.gpu
def test_glue_kernels():
    rng = np.random.default_rng(1)
    x = bf16_round(rng.standard_normal((33, 4096)).astype(np.float32) * 3)
    y = bf16_round(rng.standard_normal((33, 4096)).astype(np.float32))
    say("glue kernels")
    xn = to_host(uno.rmsnorm(to_dev(x, "bf16"), 1e-5))
    assert floored_rel_err(xn, oracle.stack.rmsnorm(x, 1e-5)) <= 1e-2
    s = to_host(uno.silu_mul(to_dev(x, "bf16"), to_dev(y, "bf16")))
    assert floored_rel_err(s, oracle.stack.silu_mul(x, y)) <= 1e-2
    r = to_host(uno.residual_add(to_dev(x, "bf16"), to_dev(y, "bf16")))
    assert floored_rel_err(r, oracle.stack.residual_add(x, y)) <= 1e-2
    # odd length exercises the scalar tail
    xo, yo = x.reshape(-1)[:1001].copy(), y.reshape(-1)[:1001].copy()
    ro = to_host(uno.residual_add(to_dev(xo, "bf16"), to_dev(yo, "bf16")))
    assert floored_rel_err(ro[None], oracle.stack.residual_add(xo, yo)[None]) <= 1e-2


@pytest.mark.gpu
@pytest.mark.parametrize("K", [4096, 8, 1032, 16384])
def test_residual_rmsnorm_fused(K):
    """The fused launch equals residual_add then rmsnorm bit for bit, in place too,
    and stays within the oracle's bound.  K = 16384 takes the re-read path."""
    rng = np.random.default_rng(K)
    M = 37
    x = bf16_round(rng.standard_normal((M, K)).astype(np.float32) * 3)
    y = bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    say(f"residual_rmsnorm K={K}")
    xd, yd = to_dev(x, "bf16"), to_dev(y, "bf16")
    s_ref = uno.residual_add(xd, yd)
    h_ref = uno.rmsnorm(s_ref, 1e-5)
    s, h = uno.residual_rmsnorm(xd, yd, 1e-5)
    assert torch.equal(s, s_ref) and torch.equal(h, h_ref)
    xin = xd.clone()
    s2, h2 = uno.residual_rmsnorm(xin, yd, 1e-5, s_out=xin)
    assert s2.data_ptr() == xin.data_ptr()
    assert torch.equal(xin, s_ref) and torch.equal(h2, h_ref)
    ref = oracle.stack.rmsnorm(oracle.stack.residual_add(x, y), 1e-5)
    assert floored_rel_err(to_host(h), ref) <= 2e-2


def _check_trace(layer, trace, gate, rows):
    for name in PROJECTIONS:
        inp, out = trace[name]
        w, a, b = (to_host(t) for t in layer[name])
        xin = to_host(inp)[rows]
        ref = oracle.gated_lora(xin, w, a, b, gate[rows], 2.0)
        err = floored_rel_err(to_host(out)[rows], ref)
        assert err <= BF16_TOL, (name, err)


@pytest.mark.gpu
@pytest.mark.parametrize("grouped", [True, False])
def test_small_stack_teacher_forced(grouped):
    shapes = (("q", 512, 512), ("k", 512, 128), ("v", 512, 128), ("o", 512, 512),
              ("gate", 512, 1024), ("up", 512, 1024), ("down", 1024, 512))
    layers = [sdev.layer_weights(shapes, 100 + 100 * i) for i in range(3)]
    gate = gate_vector(4, 16, 16)
    st = uno.GatedLoraStack(layers, to_dev(gate, "u8"), grouped=grouped)
    x0 = sdev.randn((gate.size, 512), 1.0, 7)
    say("small stack, grouped" if grouped else "small stack, one launch per projection")
    for li in range(3):
        trace = {}
        out = st.forward(x0, trace_layer=li, trace=trace)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        _check_trace(layers[li], trace, gate, np.arange(gate.size))


@pytest.mark.gpu
def test_grouped_stack_matches_ungrouped():
    """K = 512 runs unsplit in both modes, so stacking changes no sum: bitwise equal."""
    shapes = (("q", 512, 512), ("k", 512, 128), ("v", 512, 128), ("o", 512, 512),
              ("gate", 512, 1024), ("up", 512, 1024), ("down", 1024, 512))
    layers = [sdev.layer_weights(shapes, 300 + 100 * i) for i in range(2)]
    gate = gate_vector(4, 16, 16)
    x0 = sdev.randn((gate.size, 512), 1.0, 9)
    say("grouped vs ungrouped stack")
    a = uno.GatedLoraStack(layers, to_dev(gate, "u8"), grouped=True, fused=False).forward(x0).clone()
    b = uno.GatedLoraStack(layers, to_dev(gate, "u8"), grouped=False).forward(x0).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.gpu
def test_fused_stack_matches_unfused_8b_shapes():
    """Residual adds and SwiGLU in the GEMM epilogues give the unfused chain's bits
    (two layers of the 8B shapes at 32 x [16 | 16] rows, the bench's plans)."""
    wl = WORKLOADS["stack32_b32"]
    layers = [sdev.layer_weights(wl.projections, 77 + 100 * i) for i in range(2)]
    gate = gate_vector(wl.n_seq, wl.verify_rows, wl.draft_rows)
    x0 = sdev.randn((wl.rows, 4096), 1.0, 3)
    say("fused vs unfused stack, 8B shapes")
    a = uno.GatedLoraStack(layers, to_dev(gate, "u8"), fused=True).forward(x0).clone()
    b = uno.GatedLoraStack(layers, to_dev(gate, "u8"), fused=False).forward(x0).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.gpu
def test_full_stack_bench_configuration():
    """The 32-layer 8B-shaped stack at batch 32 x [16 | 16], as the bench runs it."""
    wl = WORKLOADS["stack32_b32"]
    layers = [sdev.layer_weights(wl.projections, wl.seed * 1000 + 100 * i) for i in range(wl.layers)]
    gate = gate_vector(wl.n_seq, wl.verify_rows, wl.draft_rows)
    st = uno.GatedLoraStack(layers, to_dev(gate, "u8"))
    x0 = sdev.randn((wl.rows, 4096), 1.0, wl.seed)
    rows = np.array([0, 15, 16, 31, 500, 517, 1007, 1023])
    for li in (0, wl.layers - 1):
        say("full stack, traced layer", li)
        trace = {}
        out = st.forward(x0, trace_layer=li, trace=trace)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        _check_trace(layers[li], trace, gate, rows)
