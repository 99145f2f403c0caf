"""C-ABI checks that need no GPU: the library loads, exports every function
include/uno.h declares, and rejects bad arguments on the host before any
launch (only argument combinations that fail validation are passed, so
nothing reaches the device)."""

import ctypes
import os
import subprocess

import pytest

import lossless_speculative_drafting_amd as uno
from lossless_speculative_drafting_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "uno.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x100000)      # never dereferenced: every call below fails validation first
NULL = ctypes.c_void_p(0)
STREAM = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    return uno.library()


def test_every_declared_symbol_is_exported(lib):
    declared = _lib.header_symbols(HEADER)
    assert len(declared) >= 13
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [s for s in declared if s not in exported]
    assert not missing, missing
    for s in declared:
        assert hasattr(lib, s)
    assert set(declared) == set(_lib.SIGNATURES), "binding signatures must mirror the header"


def test_version_and_status_strings(lib):
    assert lib.uno_abi_version() == 1
    assert uno.status_string(0) == "UNO_OK"
    assert uno.status_string(3) == "UNO_ERR_WORKSPACE"
    assert uno.status_string(99) == "UNO_ERR_UNKNOWN"


def _msg(lib):
    return lib.uno_last_error_message().decode()


def test_philox_validation(lib):
    assert lib.uno_philox_uniforms(0, 0, 0, -1, FAKE, STREAM) == INVALID
    assert lib.uno_philox_uniforms(0, 0, 0, 5, NULL, STREAM) == INVALID
    assert lib.uno_philox_uniforms(0, 0, 2 ** 64 - 2, 5, FAKE, STREAM) == INVALID
    assert "2^64" in _msg(lib)
    assert lib.uno_philox_uniforms(0, 0, 0, 0, NULL, STREAM) == OK   # n = 0 is a no-op


def test_gated_lora_validation(lib):
    def call(M=4, N=16, K=16, r=16, dt=0, x=FAKE, ws=FAKE, wsb=1 << 30, scale=2.0):
        return lib.uno_gated_lora_fwd(x, FAKE, FAKE, FAKE, FAKE, FAKE, M, N, K, r, scale, dt, ws, wsb, STREAM)
    assert call(dt=7) == INVALID
    assert call(N=0) == INVALID
    assert call(M=-1) == INVALID
    assert call(K=12) == UNSUPPORTED and "K % 8" in _msg(lib)
    assert call(r=300) == UNSUPPORTED
    assert call(r=12) == UNSUPPORTED
    assert call(scale=float("inf")) == INVALID
    assert call(x=NULL) == INVALID
    assert call(ws=NULL) == WORKSPACE
    assert call(wsb=16) == WORKSPACE
    assert call(ws=ctypes.c_void_p(0x100010)) == WORKSPACE   # not 256-byte aligned
    assert call(M=0, x=NULL) == OK                            # empty batch is a no-op
    assert lib.uno_gated_lora_workspace_size(2048, 4096, 4096, 128, 0) > 0
    # fp32 path: the row plan (gate-error count), then T [M, r] fp32
    assert lib.uno_gated_lora_workspace_size(24, 512, 512, 128, 1) == lib.uno_row_plan_size(24) + 24 * 128 * 4


def test_few_row_plans_through_workspace_sizes(lib, monkeypatch):
    """At 32 rows or fewer the launches take the compact 32-row tiles: the SwiGLU launch
    needs no split of K (224 tiles for 28672 interleaved columns: no workspace), a plain
    projection of 4096 columns splits K eight ways over 32 column blocks (fp32 partials of
    the plan's 64 rows); with UNO_COMPACT=0 the SwiGLU launch splits K again."""
    for var in ("UNO_GEMM_TILE", "UNO_GEMM_SPLIT", "UNO_STREAM", "UNO_COMPACT"):
        monkeypatch.delenv(var, raising=False)
    assert lib.uno_gated_gemm_swiglu_workspace_size(32, 14336, 4096, 256) == 0
    assert lib.uno_gated_gemm_workspace_size(32, 4096, 4096, 128) == 8 * 64 * 4096 * 4
    assert lib.uno_gated_gemm_workspace_size(32, 4096, 14336, 128) == 8 * 64 * 4096 * 4
    monkeypatch.setenv("UNO_COMPACT", "0")
    assert lib.uno_gated_gemm_swiglu_workspace_size(32, 14336, 4096, 256) > 0


def test_row_plan_gate_error_query(lib):
    # the plan holds a 256-byte header (gate-error count and first bad row
    # among it), the permutation over 32-row-padded segments, and the list of
    # rows with an invalid gate byte
    for M in (1, 24, 1024, 1000003):
        rows_cap = (M + 31) // 32 * 32 + 32
        need = 256 + 4 * (rows_cap + M)
        assert lib.uno_row_plan_size(M) >= need and lib.uno_row_plan_size(M) % 256 == 0
    assert lib.uno_row_plan_size(-1) == 0
    assert lib.uno_row_plan_gate_errors(NULL, FAKE, STREAM) == INVALID
    assert lib.uno_row_plan_gate_errors(FAKE, NULL, STREAM) == INVALID
    assert lib.uno_row_plan_gate_errors(ctypes.c_void_p(0x100010), FAKE, STREAM) == INVALID  # plan not 256-aligned
    assert lib.uno_row_plan_gate_errors(FAKE, ctypes.c_void_p(0x100002), STREAM) == INVALID  # out not 4-aligned


def test_grouped_gemm_and_lora_t_validation(lib):
    def call(groups=(4096, 1024, 1024), M=64, K=256, r=128, ys=None, ws=FAKE, wsb=1 << 30):
        ns = (ctypes.c_int64 * max(1, len(groups)))(*groups)
        y = ys if ys is not None else (ctypes.c_void_p * max(1, len(groups)))(*([0x100000] * len(groups)))
        return lib.uno_gated_gemm_grouped(FAKE, FAKE, FAKE, FAKE, FAKE, y, ns, len(groups), M, K, r, ws, wsb, STREAM)
    assert call(groups=()) == UNSUPPORTED
    assert call(groups=(128, 128, 128, 128, 128)) == UNSUPPORTED
    assert call(groups=(4000, 96)) == UNSUPPORTED and "multiple of 128" in _msg(lib)
    assert call(groups=(128, 0)) == INVALID
    assert call(r=12) == UNSUPPORTED
    assert call(groups=(256, 256, 256, 256), r=256, M=1 << 20) == UNSUPPORTED  # T too wide for 2^30 elements
    assert call(ys=(ctypes.c_void_p * 3)(0x100000, 0, 0x100000)) == INVALID
    assert call(ys=(ctypes.c_void_p * 3)(0x100000, 0x100008, 0x100000)) == INVALID  # misaligned output
    assert call(M=0) == OK                                      # empty batch: no launch
    # a ragged last group is accepted (the size query succeeds and clears the error)
    ns = (ctypes.c_int64 * 2)(4096, 1000)
    lib.uno_gated_gemm_grouped_workspace_size(1024, 4096, 128, ns, 2)
    assert lib.uno_last_error_message() == b""
    # T may stack several adapters: width up to 1024
    assert lib.uno_lora_t_size(1024, 384) == 1024 * 0 + ((1024 + 31) // 32 * 32 + 32) * 384 * 2
    assert lib.uno_lora_t_size(1024, 1032) == 0
    assert lib.uno_lora_down(FAKE, FAKE, FAKE, FAKE, 64, 256, 1032, 2.0, FAKE, 1 << 30, STREAM) == UNSUPPORTED
    assert lib.uno_lora_down(FAKE, FAKE, FAKE, FAKE, 64, 256, 20, 2.0, FAKE, 1 << 30, STREAM) == UNSUPPORTED


def test_block_verify_validation(lib):
    def call(B=2, L=4, V=64, nb=0, T=1.0, dt=0, tok=FAKE, ws=FAKE, wsb=1 << 30, ts=256, ds=256):
        return lib.uno_block_verify(FAKE, FAKE, ts, ds, tok, FAKE, B, L, V, nb, T, dt, FAKE, FAKE, FAKE, ws, wsb,
                                    STREAM)
    assert call(L=0) == INVALID
    assert call(L=65) == UNSUPPORTED
    assert call(L=64, nb=1) == UNSUPPORTED
    assert call(nb=2) == INVALID
    assert call(T=0.0) == UNSUPPORTED
    assert call(T=float("nan")) == UNSUPPORTED
    assert call(dt=3) == INVALID
    assert call(V=0) == INVALID
    assert call(ts=-1) == INVALID
    assert call(tok=NULL) == INVALID
    assert call(wsb=8) == WORKSPACE
    assert call(B=0, tok=NULL) == OK
    assert lib.uno_block_verify_workspace_size(64, 16, 128256, 0) > 0
    assert lib.uno_block_verify_workspace_size(64, 65, 128256, 0) == 0


def test_block_verify_early_validation(lib):
    assert lib.uno_block_verify_early_workspace_size(64, 16, 128256, 0) >= lib.uno_block_verify_workspace_size(64, 16, 128256, 0) > 0
    assert lib.uno_block_verify_early_workspace_size(64, 65, 128256, 0) == 0
    args = (FAKE, FAKE, 0, 0, FAKE, FAKE, 4, 8, 64, 0, 1.0, 0)
    tail = (FAKE, FAKE, FAKE, FAKE, 1 << 30, STREAM)
    assert lib.uno_block_verify_early(*args, 0, *tail) == INVALID        # chunk < 1
    assert lib.uno_block_verify_early(*args, 65, *tail) == INVALID       # chunk > 64
    assert lib.uno_block_verify_early(FAKE, FAKE, 0, 0, FAKE, FAKE, 4, 8, 64, 0, -1.0, 0, 4, *tail) != OK
    assert lib.uno_block_verify_early(FAKE, FAKE, 0, 0, FAKE, FAKE, 4, 8, 64, 0, 1.0, 0, 4,
                                      FAKE, FAKE, FAKE, FAKE, 4, STREAM) == WORKSPACE
    assert lib.uno_block_verify_early(NULL, NULL, 0, 0, NULL, NULL, 0, 8, 64, 0, 1.0, 0, 4,
                                      NULL, NULL, NULL, NULL, 0, STREAM) == OK


def test_draft_sample_and_glue_validation(lib):
    assert lib.uno_draft_sample(FAKE, 0, FAKE, 2, 0, 64, 1.0, 0, FAKE, FAKE, 1 << 30, STREAM) == INVALID
    assert lib.uno_draft_sample(FAKE, 0, FAKE, 2, 4, 64, -1.0, 0, FAKE, FAKE, 1 << 30, STREAM) == UNSUPPORTED
    assert lib.uno_draft_sample(FAKE, 0, FAKE, 2, 4, 64, 1.0, 0, FAKE, FAKE, 4, STREAM) == WORKSPACE
    assert lib.uno_rmsnorm(FAKE, FAKE, 4, 12, 1e-5, 0, STREAM) == UNSUPPORTED
    assert lib.uno_rmsnorm(FAKE, FAKE, 4, 16, 1e-5, 1, STREAM) == UNSUPPORTED
    assert lib.uno_rmsnorm(FAKE, FAKE, 4, 16, -1.0, 0, STREAM) == INVALID
    assert lib.uno_silu_mul(FAKE, NULL, FAKE, 16, 0, STREAM) == INVALID
    assert lib.uno_residual_add(FAKE, FAKE, ctypes.c_void_p(0x100004), 16, 0, STREAM) == INVALID
    assert lib.uno_silu_mul(NULL, NULL, NULL, 0, 0, STREAM) == OK
    assert lib.uno_residual_rmsnorm(FAKE, FAKE, FAKE, FAKE, 4, 12, 1e-5, 0, STREAM) == UNSUPPORTED
    assert lib.uno_residual_rmsnorm(FAKE, FAKE, FAKE, FAKE, 4, 16, 1e-5, 1, STREAM) == UNSUPPORTED
    assert lib.uno_residual_rmsnorm(FAKE, FAKE, FAKE, FAKE, 4, 16, float("nan"), 0, STREAM) == INVALID
    assert lib.uno_residual_rmsnorm(FAKE, NULL, FAKE, FAKE, 4, 16, 1e-5, 0, STREAM) == INVALID
    assert lib.uno_residual_rmsnorm(FAKE, FAKE, FAKE, ctypes.c_void_p(0x100004), 4, 16, 1e-5, 0, STREAM) == INVALID
    assert lib.uno_residual_rmsnorm(NULL, NULL, NULL, NULL, 0, 16, 1e-5, 0, STREAM) == OK


def test_lm_head_verify_validation(lib):
    assert lib.uno_lm_head_verify_workspace_size(32, 16, 128256, 4096, 1) > 0
    assert lib.uno_lm_head_verify_workspace_size(32, 65, 128256, 4096, 0) == 0   # L > 64
    assert lib.uno_lm_head_verify_workspace_size(32, 16, 128256, 4100, 0) == 0   # K % 8 != 0
    assert lib.uno_lm_head_verify_workspace_size(32, 16, 1 << 20, 4096, 0) == 0  # V K >= 2^30
    args = (FAKE, FAKE, 4, 8, 1024, 256)
    outs = (FAKE, FAKE, FAKE, FAKE, FAKE, NULL)   # tokens, uniforms, three outputs, logits
    assert lib.uno_lm_head_verify(*args, 2, 1.0, *outs, FAKE, 1 << 30, STREAM) == INVALID       # has_bonus
    assert lib.uno_lm_head_verify(*args, 0, 0.0, *outs, FAKE, 1 << 30, STREAM) == UNSUPPORTED   # T
    assert lib.uno_lm_head_verify(FAKE, FAKE, 4, 64, 1024, 256, 1, 1.0, *outs, FAKE, 1 << 30, STREAM) == UNSUPPORTED
    assert lib.uno_lm_head_verify(FAKE, FAKE, 4, 8, 1024, 12, 0, 1.0, *outs, FAKE, 1 << 30, STREAM) == UNSUPPORTED
    assert lib.uno_lm_head_verify(NULL, FAKE, 4, 8, 1024, 256, 0, 1.0, *outs, FAKE, 1 << 30, STREAM) == INVALID
    assert lib.uno_lm_head_verify(ctypes.c_void_p(0x100008), FAKE, 4, 8, 1024, 256, 0, 1.0, *outs, FAKE, 1 << 30,
                                  STREAM) == INVALID                                        # alignment
    assert lib.uno_lm_head_verify(*args, 0, 1.0, *outs, FAKE, 4, STREAM) == WORKSPACE
    assert lib.uno_lm_head_verify(NULL, NULL, 0, 8, 1024, 256, 0, 1.0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                                  STREAM) == OK                                             # B = 0


def test_tree_verify_validation(lib):
    assert lib.uno_tree_verify_workspace_size(32, 64, 128256) > 0
    assert lib.uno_tree_verify_workspace_size(32, 0, 128256) == 0
    assert lib.uno_tree_verify_workspace_size(32, 4097, 128256) == 0
    outs = (FAKE, FAKE, FAKE, FAKE)
    assert lib.uno_tree_verify(FAKE, 0, FAKE, FAKE, FAKE, 4, 0, 64, 1.0, 0, *outs, FAKE, 1 << 30, STREAM) == UNSUPPORTED
    assert lib.uno_tree_verify(FAKE, 0, FAKE, FAKE, FAKE, 4, 8, 64, -1.0, 0, *outs, FAKE, 1 << 30, STREAM) == UNSUPPORTED
    assert lib.uno_tree_verify(FAKE, 0, FAKE, FAKE, FAKE, 4, 8, 64, 1.0, 7, *outs, FAKE, 1 << 30, STREAM) == INVALID
    assert lib.uno_tree_verify(FAKE, -1, FAKE, FAKE, FAKE, 4, 8, 64, 1.0, 0, *outs, FAKE, 1 << 30, STREAM) == INVALID
    assert lib.uno_tree_verify(FAKE, 0, NULL, FAKE, FAKE, 4, 8, 64, 1.0, 0, *outs, FAKE, 1 << 30, STREAM) == INVALID
    assert lib.uno_tree_verify(ctypes.c_void_p(0x100001), 0, FAKE, FAKE, FAKE, 4, 8, 64, 1.0, 0, *outs, FAKE, 1 << 30,
                               STREAM) == INVALID
    assert lib.uno_tree_verify(FAKE, 0, FAKE, FAKE, FAKE, 4, 8, 64, 1.0, 0, *outs, FAKE, 4, STREAM) == WORKSPACE
    assert lib.uno_tree_verify(NULL, 0, NULL, NULL, NULL, 0, 8, 64, 1.0, 0, NULL, NULL, NULL, NULL, NULL, 0,
                               STREAM) == OK
