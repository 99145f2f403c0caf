"""ctypes binding to libuno.so: argument marshalling only.

Every function takes torch tensors that already live on the GPU, passes their
device pointers, sizes and the current HIP stream to the C ABI declared in
include/uno.h, and returns tensors the caller owns.  Workspaces are plain
torch byte tensors sized by the library's own *_workspace_size queries.  No
computation happens here; if the shared library is missing the import fails.
"""

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("UNO_LIB", os.path.join(_HERE, "libuno.so"))

UNO_BF16 = 0
UNO_F32 = 1

_c_int32, _c_int64, _c_uint64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
_c_size, _c_float, _c_ptr = ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p

# name: (restype, argtypes) -- mirrors include/uno.h
SIGNATURES = {
    "uno_abi_version": (_c_int32, []),
    "uno_status_string": (ctypes.c_char_p, [_c_int32]),
    "uno_last_error_message": (ctypes.c_char_p, []),
    "uno_philox_uniforms": (_c_int32, [_c_uint64, _c_uint64, _c_uint64, _c_int64, _c_ptr, _c_ptr]),
    "uno_gated_lora_workspace_size": (_c_size, [_c_int64, _c_int64, _c_int64, _c_int32, _c_int32]),
    "uno_gated_lora_fwd": (_c_int32, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_int64, _c_int64,
                                      _c_int64, _c_int32, _c_float, _c_int32, _c_ptr, _c_size, _c_ptr]),
    "uno_row_plan_size": (_c_size, [_c_int64]),
    "uno_segment_rows": (_c_int32, [_c_ptr, _c_int64, _c_ptr, _c_size, _c_ptr]),
    "uno_row_plan_gate_errors": (_c_int32, [_c_ptr, _c_ptr, _c_ptr]),
    "uno_lora_t_size": (_c_size, [_c_int64, _c_int32]),
    "uno_lora_down_workspace_size": (_c_size, [_c_int64, _c_int64, _c_int32]),
    "uno_lora_down": (_c_int32, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_int64, _c_int64, _c_int32, _c_float, _c_ptr,
                                 _c_size, _c_ptr]),
    "uno_gated_gemm_workspace_size": (_c_size, [_c_int64, _c_int64, _c_int64, _c_int32]),
    "uno_gated_gemm": (_c_int32, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_int64, _c_int64, _c_int64,
                                  _c_int32, _c_ptr, _c_size, _c_ptr]),
    "uno_gated_gemm_residual_workspace_size": (_c_size, [_c_int64, _c_int64, _c_int64, _c_int32]),
    "uno_gated_gemm_residual": (_c_int32, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_int64, _c_int64,
                                           _c_int64, _c_int32, _c_ptr, _c_size, _c_ptr]),
    "uno_gated_gemm_swiglu_workspace_size": (_c_size, [_c_int64, _c_int64, _c_int64, _c_int32]),
    "uno_gated_gemm_swiglu": (_c_int32, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_int64, _c_int64,
                                         _c_int64, _c_int32, _c_ptr, _c_size, _c_ptr]),
    "uno_swiglu_pack": (_c_int32, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_int64, _c_int64, _c_int32, _c_ptr, _c_ptr,
                                   _c_ptr]),
    "uno_gated_gemm_grouped_workspace_size": (_c_size, [_c_int64, _c_int64, _c_int32, _c_ptr, _c_int32]),
    "uno_gated_gemm_grouped": (_c_int32, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_int32,
                                          _c_int64, _c_int64, _c_int32, _c_ptr, _c_size, _c_ptr]),
    "uno_block_verify_workspace_size": (_c_size, [_c_int64, _c_int32, _c_int64, _c_int32]),
    "uno_block_verify": (_c_int32, [_c_ptr, _c_ptr, _c_int64, _c_int64, _c_ptr, _c_ptr, _c_int64, _c_int32,
                                    _c_int64, _c_int32, _c_float, _c_int32, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                    _c_size, _c_ptr]),
    "uno_block_verify_noalloc_max_bytes": (_c_size, []),
    "uno_block_verify_noalloc": (_c_int32, [_c_ptr, _c_ptr, _c_int64, _c_int64, _c_ptr, _c_ptr, _c_int64, _c_int32,
                                            _c_int64, _c_int32, _c_float, _c_int32, _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "uno_block_verify_early_workspace_size": (_c_size, [_c_int64, _c_int32, _c_int64, _c_int32]),
    "uno_block_verify_early": (_c_int32, [_c_ptr, _c_ptr, _c_int64, _c_int64, _c_ptr, _c_ptr, _c_int64, _c_int32,
                                          _c_int64, _c_int32, _c_float, _c_int32, _c_int32, _c_ptr, _c_ptr, _c_ptr,
                                          _c_ptr, _c_size, _c_ptr]),
    "uno_draft_sample_workspace_size": (_c_size, [_c_int64, _c_int32, _c_int64]),
    "uno_draft_sample": (_c_int32, [_c_ptr, _c_int64, _c_ptr, _c_int64, _c_int32, _c_int64, _c_float,
                                    _c_int32, _c_ptr, _c_ptr, _c_size, _c_ptr]),
    "uno_tree_verify_workspace_size": (_c_size, [_c_int64, _c_int32, _c_int64]),
    "uno_tree_verify": (_c_int32, [_c_ptr, _c_int64, _c_ptr, _c_ptr, _c_ptr, _c_int64, _c_int32, _c_int64, _c_float,
                                   _c_int32, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr]),
    "uno_lm_head_verify_workspace_size": (_c_size, [_c_int64, _c_int32, _c_int64, _c_int64, _c_int32]),
    "uno_lm_head_verify": (_c_int32, [_c_ptr, _c_ptr, _c_int64, _c_int32, _c_int64, _c_int64, _c_int32, _c_float,
                                      _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr]),
    "uno_rmsnorm": (_c_int32, [_c_ptr, _c_ptr, _c_int64, _c_int64, _c_float, _c_int32, _c_ptr]),
    "uno_silu_mul": (_c_int32, [_c_ptr, _c_ptr, _c_ptr, _c_int64, _c_int32, _c_ptr]),
    "uno_residual_add": (_c_int32, [_c_ptr, _c_ptr, _c_ptr, _c_int64, _c_int32, _c_ptr]),
    "uno_residual_rmsnorm": (_c_int32, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_int64, _c_int64, _c_float, _c_int32,
                                        _c_ptr]),
}


class UnoError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libuno.so not found at {LIB_PATH}; build it with "
            "`python lossless_speculative_drafting_amd/build.py` (there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def library():
    return _lib


def status_string(status):
    return _lib.uno_status_string(status).decode()


def _check(status):
    if status != 0:
        raise UnoError(status, _lib.uno_last_error_message().decode())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return UNO_BF16
    if dt == torch.float32:
        return UNO_F32
    raise TypeError(f"unsupported dtype {dt}")


def _need_cuda(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


class Workspace:
    """A grow-only device byte buffer reused across calls.

    Calls that share a Workspace must not overlap in time (the library's
    rule for any workspace).  The buffer is marked as used on the stream of
    each call, so that when it grows the caching allocator does not hand the
    old buffer out again while work on that stream may still read it.
    """

    def __init__(self, device=None):
        self.device = device
        self.buf = None

    def get(self, nbytes, stream=None):
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(int(nbytes), dtype=torch.uint8, device=self.device or "cuda")
        if stream is not None:
            self.buf.record_stream(stream)
        return self.buf


_default_ws = {}


def _workspace(ws, nbytes, device, stream=None):
    """The caller's workspace, or a default one per (device, stream)."""
    s = torch.cuda.current_stream(device) if stream is None else stream
    if ws is None:
        key = (device.index if device.index is not None else torch.cuda.current_device(), s.cuda_stream)
        ws = _default_ws.setdefault(key, Workspace(device))
    return ws.get(nbytes, s)


# ------------------------------------------------------------------ Philox

def philox_uniforms(seed, stream_id, offset, n, out=None, device="cuda", stream=None):
    """float32 uniforms for Philox words offset .. offset+n-1 of (seed, stream_id)."""
    if out is None:
        out = torch.empty(int(n), dtype=torch.float32, device=device)
    _need_cuda(out)
    if out.numel() < n or out.dtype != torch.float32:
        raise ValueError("out must be a float32 tensor with at least n elements")
    _check(_lib.uno_philox_uniforms(int(seed), int(stream_id), int(offset), int(n), _ptr(out), _stream(stream)))
    return out


# ------------------------------------------------------------------ gated LoRA

def gated_lora_workspace_size(M, N, K, r, dtype):
    return int(_lib.uno_gated_lora_workspace_size(M, N, K, r, _dtype_code(dtype)))


def gated_lora_fwd(x, w, lora_a, lora_b, gate, scale=2.0, out=None, workspace=None, stream=None,
                   gate_errors=None):
    """y = x W_AR + gate * scale * (x A) B with storage w [N,K], lora_a [r,K], lora_b [N,r].

    Rows whose gate byte is neither 0 nor 1 come out as NaN; with
    gate_errors (a device int32 tensor of 2 elements) the call also writes
    {number of such rows, first such row or -1} there.
    """
    _need_cuda(x, w, lora_a, lora_b, gate)
    M, K = x.shape
    N = w.shape[0]
    r = lora_a.shape[0]
    if w.shape != (N, K) or lora_a.shape != (r, K) or lora_b.shape != (N, r) or gate.shape != (M,):
        raise ValueError("shape mismatch: x [M,K], w [N,K], lora_a [r,K], lora_b [N,r], gate [M]")
    if gate.dtype != torch.uint8:
        raise TypeError("gate must be uint8")
    if not (x.dtype == w.dtype == lora_a.dtype == lora_b.dtype):
        raise TypeError("x, w, lora_a and lora_b must share a dtype")
    dt = _dtype_code(x.dtype)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _need_cuda(out)
    need = int(_lib.uno_gated_lora_workspace_size(M, N, K, r, dt))
    ws = _workspace(workspace, need, x.device, stream)
    _check(_lib.uno_gated_lora_fwd(_ptr(x), _ptr(w), _ptr(lora_a), _ptr(lora_b), _ptr(gate), _ptr(out),
                                   M, N, K, r, float(scale), dt, _ptr(ws), need, _stream(stream)))
    if gate_errors is not None:
        _gate_errors_into(ws, gate_errors, stream)
    return out


def _gate_errors_into(plan_buf, out, stream):
    _need_cuda(out)
    if out.dtype != torch.int32 or out.numel() < 2:
        raise ValueError("gate_errors must be a device int32 tensor of 2 elements")
    _check(_lib.uno_row_plan_gate_errors(_ptr(plan_buf), _ptr(out), _stream(stream)))
    return out


class RowPlan:
    """Device row plan for a gate vector (uno_segment_rows), reusable across projections."""

    def __init__(self, gate, stream=None):
        _need_cuda(gate)
        if gate.dtype != torch.uint8 or gate.dim() != 1:
            raise TypeError("gate must be a 1-D uint8 tensor")
        self.M = gate.shape[0]
        self.gate = gate
        self.nbytes = int(_lib.uno_row_plan_size(self.M))
        self.buf = torch.empty(max(self.nbytes, 256), dtype=torch.uint8, device=gate.device)
        _check(_lib.uno_segment_rows(_ptr(gate), self.M, _ptr(self.buf), self.nbytes, _stream(stream)))

    def gate_errors(self, out=None, stream=None):
        """Device int32 [2]: rows whose gate byte is neither 0 nor 1, and the first such row (-1 if none)."""
        if out is None:
            out = torch.empty(2, dtype=torch.int32, device=self.buf.device)
        return _gate_errors_into(self.buf, out, stream)


def lora_t_size(M, r):
    return int(_lib.uno_lora_t_size(M, r))


def lora_down(x, lora_a, plan, scale=2.0, t=None, workspace=None, stream=None):
    """T = scale * (x A) on the plan's draft rows (bf16, plan order); returns the T buffer."""
    _need_cuda(x, lora_a)
    M, K = x.shape
    r = lora_a.shape[0]
    if lora_a.shape != (r, K) or plan.M != M:
        raise ValueError("shape mismatch: x [M,K], lora_a [r,K], plan over M rows")
    if t is None:
        t = torch.empty(lora_t_size(M, r) // 2, dtype=torch.bfloat16, device=x.device)
    need = int(_lib.uno_lora_down_workspace_size(M, K, r))
    ws = _workspace(workspace, need, x.device, stream)
    _check(_lib.uno_lora_down(_ptr(x), _ptr(lora_a), _ptr(plan.buf), _ptr(t), M, K, r, float(scale), _ptr(ws), need,
                              _stream(stream)))
    return t


def gated_gemm(x, w, t, lora_b, plan, out=None, workspace=None, stream=None):
    """y = x W_AR + T B on the plan's draft rows, T from lora_down with the same plan."""
    _need_cuda(x, w, t, lora_b)
    M, K = x.shape
    N = w.shape[0]
    r = lora_b.shape[1]
    if w.shape != (N, K) or lora_b.shape != (N, r) or plan.M != M:
        raise ValueError("shape mismatch: x [M,K], w [N,K], lora_b [N,r], plan over M rows")
    if t.numel() * t.element_size() < lora_t_size(M, r):
        raise ValueError("t buffer too small")
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    need = int(_lib.uno_gated_gemm_workspace_size(M, N, K, r))
    ws = _workspace(workspace, need, x.device, stream)
    _check(_lib.uno_gated_gemm(_ptr(x), _ptr(w), _ptr(t), _ptr(lora_b), _ptr(plan.buf), _ptr(out), M, N, K, r,
                               _ptr(ws), need, _stream(stream)))
    return out


def gated_gemm_grouped(x, w, t, lora_b, plan, group_n, outs=None, workspace=None, stream=None):
    """Several projections of the same x in one launch (uno_gated_gemm_grouped).

    w [N, K] and lora_b [N, r] stack the groups' rows (N = sum(group_n)); t is
    lora_down over the stacked A matrices (width len(group_n) * r).  Returns
    one [M, group_n[g]] output per group (outs, if given).
    """
    _need_cuda(x, w, t, lora_b)
    M, K = x.shape
    group_n = [int(n) for n in group_n]
    G = len(group_n)
    N = sum(group_n)
    r = lora_b.shape[1]
    if w.shape != (N, K) or lora_b.shape != (N, r) or plan.M != M:
        raise ValueError("shape mismatch: x [M,K], w [N,K], lora_b [N,r] with N = sum(group_n), plan over M rows")
    if t.numel() * t.element_size() < lora_t_size(M, r * G):
        raise ValueError("t buffer too small")
    if outs is None:
        outs = [torch.empty((M, n), dtype=x.dtype, device=x.device) for n in group_n]
    if len(outs) != G or any(o.shape != (M, n) or not o.is_contiguous() for o, n in zip(outs, group_n)):
        raise ValueError("outs must be contiguous [M, group_n[g]] tensors")
    ns = (ctypes.c_int64 * G)(*group_n)
    ys = (ctypes.c_void_p * G)(*[_ptr(o) for o in outs])
    need = int(_lib.uno_gated_gemm_grouped_workspace_size(M, K, r, ns, G))  # 0 also on bad shapes: the call reports those
    ws = _workspace(workspace, need, x.device, stream)
    _check(_lib.uno_gated_gemm_grouped(_ptr(x), _ptr(w), _ptr(t), _ptr(lora_b), _ptr(plan.buf), ys, ns, G, M, K, r,
                                       _ptr(ws), need, _stream(stream)))
    return outs


def gated_gemm_residual(x, w, t, lora_b, plan, y, workspace=None, stream=None):
    """y += x W_AR + T B on the plan's draft rows (uno_gated_gemm_residual); returns y."""
    _need_cuda(x, w, t, lora_b, y)
    M, K = x.shape
    N = w.shape[0]
    r = lora_b.shape[1]
    if w.shape != (N, K) or lora_b.shape != (N, r) or y.shape != (M, N) or plan.M != M or not y.is_contiguous():
        raise ValueError("shape mismatch: x [M,K], w [N,K], lora_b [N,r], y [M,N] contiguous, plan over M rows")
    if t.numel() * t.element_size() < lora_t_size(M, r):
        raise ValueError("t buffer too small")
    need = int(_lib.uno_gated_gemm_residual_workspace_size(M, N, K, r))
    ws = _workspace(workspace, need, x.device, stream)
    _check(_lib.uno_gated_gemm_residual(_ptr(x), _ptr(w), _ptr(t), _ptr(lora_b), _ptr(plan.buf), _ptr(y), M, N, K,
                                        r, _ptr(ws), need, _stream(stream)))
    return y


def swiglu_pack(w_gate, w_up, b_gate, b_up, stream=None):
    """(w_packed [2N, K], b_packed [2N, 2r]) for gated_gemm_swiglu (uno_swiglu_pack)."""
    _need_cuda(w_gate, w_up, b_gate, b_up)
    N, K = w_gate.shape
    r = b_gate.shape[1]
    if w_up.shape != (N, K) or b_gate.shape != (N, r) or b_up.shape != (N, r):
        raise ValueError("shape mismatch: w_gate, w_up [N,K]; b_gate, b_up [N,r]")
    w_p = torch.empty((2 * N, K), dtype=w_gate.dtype, device=w_gate.device)
    b_p = torch.empty((2 * N, 2 * r), dtype=w_gate.dtype, device=w_gate.device)
    _check(_lib.uno_swiglu_pack(_ptr(w_gate), _ptr(w_up), _ptr(b_gate), _ptr(b_up), N, K, r, _ptr(w_p), _ptr(b_p),
                                _stream(stream)))
    return w_p, b_p


def gated_gemm_swiglu(x, w_packed, t, b_packed, plan, out=None, workspace=None, stream=None):
    """act = silu(x W_gate + ...) * (x W_up + ...) from swiglu_pack weights (uno_gated_gemm_swiglu)."""
    _need_cuda(x, w_packed, t, b_packed)
    M, K = x.shape
    N2 = w_packed.shape[0]
    rt = b_packed.shape[1]
    if w_packed.shape != (N2, K) or b_packed.shape != (N2, rt) or N2 % 2 or plan.M != M:
        raise ValueError("shape mismatch: x [M,K], w_packed [2N,K], b_packed [2N,rt], plan over M rows")
    if t.numel() * t.element_size() < lora_t_size(M, rt):
        raise ValueError("t buffer too small")
    Nh = N2 // 2
    if out is None:
        out = torch.empty((M, Nh), dtype=x.dtype, device=x.device)
    if out.shape != (M, Nh) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] tensor")
    need = int(_lib.uno_gated_gemm_swiglu_workspace_size(M, Nh, K, rt))
    ws = _workspace(workspace, need, x.device, stream)
    _check(_lib.uno_gated_gemm_swiglu(_ptr(x), _ptr(w_packed), _ptr(t), _ptr(b_packed), _ptr(plan.buf), _ptr(out), M,
                                      Nh, K, rt, _ptr(ws), need, _stream(stream)))
    return out


# ------------------------------------------------------------------ verification

def block_verify_workspace_size(B, L, V, has_bonus=False):
    return int(_lib.uno_block_verify_workspace_size(B, L, V, int(bool(has_bonus))))


def block_verify_early_workspace_size(B, L, V, has_bonus=False):
    return int(_lib.uno_block_verify_early_workspace_size(B, L, V, int(bool(has_bonus))))


def tree_verify_workspace_size(B, N, V):
    return int(_lib.uno_tree_verify_workspace_size(B, N, V))


def tree_verify(node_logits, parents, tokens, uniforms, temperature=1.0, outputs=None, workspace=None, stream=None):
    """Verify B candidate trees of N nodes (uno_tree_verify).

    node_logits [B, N, V] (bf16 or float32), parents / tokens int32 [B, N],
    uniforms float32 [B, N].  Returns (n_accepted [B], out_tokens [B, N],
    n_emitted [B], last_node [B]) int32 tensors.
    """
    _need_cuda(node_logits, parents, tokens, uniforms)
    B, N, V = node_logits.shape
    if parents.shape != (B, N) or tokens.shape != (B, N) or uniforms.shape != (B, N):
        raise ValueError("parents, tokens and uniforms must be [B, N]")
    if parents.dtype != torch.int32 or tokens.dtype != torch.int32 or uniforms.dtype != torch.float32:
        raise TypeError("parents and tokens must be int32, uniforms float32")
    for t in (node_logits, parents, tokens, uniforms):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    dev = node_logits.device
    if outputs is None:
        outputs = (torch.empty(B, dtype=torch.int32, device=dev), torch.empty((B, N), dtype=torch.int32, device=dev),
                   torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev))
    n_acc, out_tok, n_emit, last = outputs
    need = int(_lib.uno_tree_verify_workspace_size(B, N, V))
    ws = _workspace(workspace, need, dev, stream)
    _check(_lib.uno_tree_verify(_ptr(node_logits), N * V, _ptr(parents), _ptr(tokens), _ptr(uniforms), int(B), int(N),
                                int(V), float(temperature), _dtype_code(node_logits.dtype), _ptr(n_acc), _ptr(out_tok),
                                _ptr(n_emit), _ptr(last), _ptr(ws), need, _stream(stream)))
    return n_acc, out_tok, n_emit, last


def lm_head_verify_workspace_size(B, L, V, K, has_bonus=False):
    return int(_lib.uno_lm_head_verify_workspace_size(B, L, V, K, int(bool(has_bonus))))


def lm_head_verify(hidden, w_lm, draft_tokens, uniforms, temperature=1.0, has_bonus=False, logits=None,
                   outputs=None, workspace=None, stream=None):
    """The LM head with the verification statistics in its epilogue, then block verification.

    hidden: bf16 [B*(L+has_bonus) + B*L, K] (target rows of every sequence,
    then draft rows); w_lm: bf16 [V, K]; draft_tokens int32 [B, L]; uniforms
    float32 [B, L+1].  logits: None (no logit row is stored; the redraw rows
    are recomputed) or a bf16 [rows, V] tensor that receives the logits.
    Returns (n_accepted [B], out_tokens [B, L+1], n_emitted [B]) int32 tensors.
    """
    _need_cuda(hidden, w_lm, draft_tokens, uniforms)
    if hidden.dtype != torch.bfloat16 or w_lm.dtype != torch.bfloat16:
        raise TypeError("hidden and w_lm must be bfloat16")
    if draft_tokens.dtype != torch.int32 or uniforms.dtype != torch.float32:
        raise TypeError("draft_tokens must be int32 and uniforms float32")
    B, L = draft_tokens.shape
    V, K = w_lm.shape
    nb = 1 if has_bonus else 0
    rows = B * (L + nb) + B * L
    if hidden.shape != (rows, K) or not hidden.is_contiguous() or not w_lm.is_contiguous():
        raise ValueError(f"hidden must be contiguous [{rows}, {K}] and w_lm contiguous [V, K]")
    if uniforms.numel() < B * (L + 1) or not draft_tokens.is_contiguous() or not uniforms.is_contiguous():
        raise ValueError("uniforms must hold B*(L+1) values; tokens and uniforms contiguous")
    if logits is not None and (logits.dtype != torch.bfloat16 or logits.shape != (rows, V)
                               or not logits.is_contiguous()):
        raise ValueError(f"logits must be a contiguous bf16 [{rows}, {V}] tensor")
    dev = hidden.device
    if outputs is None:
        outputs = (torch.empty(B, dtype=torch.int32, device=dev),
                   torch.empty((B, L + 1), dtype=torch.int32, device=dev),
                   torch.empty(B, dtype=torch.int32, device=dev))
    n_acc, out_tok, n_emit = outputs
    need = int(_lib.uno_lm_head_verify_workspace_size(B, L, V, K, nb))
    ws = _workspace(workspace, need, dev, stream)
    _check(_lib.uno_lm_head_verify(_ptr(hidden), _ptr(w_lm), int(B), int(L), int(V), int(K), nb, float(temperature),
                                   _ptr(draft_tokens), _ptr(uniforms), _ptr(n_acc), _ptr(out_tok), _ptr(n_emit),
                                   _ptr(logits), _ptr(ws), need, _stream(stream)))
    return n_acc, out_tok, n_emit


def block_verify(target_logits, draft_logits, draft_tokens, uniforms, temperature=1.0, has_bonus=False,
                 B=None, L=None, V=None, target_seq_stride=None, draft_seq_stride=None,
                 outputs=None, workspace=None, stream=None, early_chunk=None, noalloc=False):
    """Verify one drafted block per sequence.

    By default target_logits is [B, L + has_bonus, V] and draft_logits [B, L, V]
    (a leading dimension of 1 broadcasts with stride 0).  Explicit B, L, V and
    strides (in elements) address logits inside a larger buffer.  early_chunk
    selects the early-exit verifier (uno_block_verify_early) with that many
    positions per chunk; its outputs are the same.  noalloc selects
    uno_block_verify_noalloc (the library's own scratch, no workspace; pass
    outputs to allocate nothing here either).
    Returns (n_accepted [B], out_tokens [B, L+1], n_emitted [B]) int32 tensors.
    """
    _need_cuda(target_logits, draft_logits, draft_tokens, uniforms)
    nb = 1 if has_bonus else 0
    if B is None:
        B, L = draft_tokens.shape
    if V is None:
        V = target_logits.shape[-1]
    if target_seq_stride is None:
        target_seq_stride = 0 if target_logits.shape[0] == 1 and B != 1 else (L + nb) * V
    if draft_seq_stride is None:
        draft_seq_stride = 0 if draft_logits.shape[0] == 1 and B != 1 else L * V
    if target_logits.dtype != draft_logits.dtype:
        raise TypeError("target and draft logits must share a dtype")
    if draft_tokens.dtype != torch.int32 or uniforms.dtype != torch.float32:
        raise TypeError("draft_tokens must be int32 and uniforms float32")
    if draft_tokens.numel() < B * L or uniforms.numel() < B * (L + 1):
        raise ValueError("draft_tokens must hold B*L and uniforms B*(L+1) values")
    for t, stride, rows in ((target_logits, target_seq_stride, L + nb), (draft_logits, draft_seq_stride, L)):
        if B > 0 and (B - 1) * stride + rows * V > t.numel():
            raise ValueError("logit buffer too small for the given B, L, V and stride")
    dev = target_logits.device
    if outputs is None:
        outputs = (torch.empty(B, dtype=torch.int32, device=dev),
                   torch.empty((B, L + 1), dtype=torch.int32, device=dev),
                   torch.empty(B, dtype=torch.int32, device=dev))
    n_acc, out_tok, n_emit = outputs
    if noalloc:
        if early_chunk is not None or workspace is not None:
            raise ValueError("the no-allocation verifier takes neither early_chunk nor a workspace")
        _check(_lib.uno_block_verify_noalloc(_ptr(target_logits), _ptr(draft_logits), int(target_seq_stride),
                                             int(draft_seq_stride), _ptr(draft_tokens), _ptr(uniforms), int(B),
                                             int(L), int(V), nb, float(temperature),
                                             _dtype_code(target_logits.dtype), _ptr(n_acc), _ptr(out_tok),
                                             _ptr(n_emit), _stream(stream)))
    elif early_chunk is None:
        need = int(_lib.uno_block_verify_workspace_size(B, L, V, nb))
        ws = _workspace(workspace, need, dev, stream)
        _check(_lib.uno_block_verify(_ptr(target_logits), _ptr(draft_logits), int(target_seq_stride),
                                     int(draft_seq_stride), _ptr(draft_tokens), _ptr(uniforms), int(B), int(L),
                                     int(V), nb, float(temperature), _dtype_code(target_logits.dtype),
                                     _ptr(n_acc), _ptr(out_tok), _ptr(n_emit), _ptr(ws), need, _stream(stream)))
    else:
        need = int(_lib.uno_block_verify_early_workspace_size(B, L, V, nb))
        ws = _workspace(workspace, need, dev, stream)
        _check(_lib.uno_block_verify_early(_ptr(target_logits), _ptr(draft_logits), int(target_seq_stride),
                                           int(draft_seq_stride), _ptr(draft_tokens), _ptr(uniforms), int(B),
                                           int(L), int(V), nb, float(temperature),
                                           _dtype_code(target_logits.dtype), int(early_chunk), _ptr(n_acc),
                                           _ptr(out_tok), _ptr(n_emit), _ptr(ws), need, _stream(stream)))
    return n_acc, out_tok, n_emit


def draft_sample_workspace_size(B, L, V):
    return int(_lib.uno_draft_sample_workspace_size(B, L, V))


def draft_sample(draft_logits, uniforms, temperature=1.0, B=None, L=None, V=None, seq_stride=None,
                 out=None, workspace=None, stream=None):
    """One token per drafted row from softmax(d / T) by inverse CDF; returns int32 [B, L]."""
    _need_cuda(draft_logits, uniforms)
    if B is None:
        B, L, V = draft_logits.shape
    if seq_stride is None:
        seq_stride = L * V
    if uniforms.dtype != torch.float32 or uniforms.numel() < B * L:
        raise ValueError("uniforms must be float32 with B*L values")
    if B > 0 and (B - 1) * seq_stride + L * V > draft_logits.numel():
        raise ValueError("logit buffer too small for the given B, L, V and stride")
    if out is None:
        out = torch.empty((B, L), dtype=torch.int32, device=draft_logits.device)
    need = int(_lib.uno_draft_sample_workspace_size(B, L, V))
    ws = _workspace(workspace, need, draft_logits.device, stream)
    _check(_lib.uno_draft_sample(_ptr(draft_logits), int(seq_stride), _ptr(uniforms), int(B), int(L), int(V),
                                 float(temperature), _dtype_code(draft_logits.dtype), _ptr(out), _ptr(ws), need,
                                 _stream(stream)))
    return out


# ------------------------------------------------------------------ glue

def rmsnorm(x, eps=1e-5, out=None, stream=None):
    _need_cuda(x)
    M, K = x.shape
    out = torch.empty_like(x) if out is None else out
    _check(_lib.uno_rmsnorm(_ptr(x), _ptr(out), M, K, float(eps), _dtype_code(x.dtype), _stream(stream)))
    return out


def silu_mul(gate, up, out=None, stream=None):
    _need_cuda(gate, up)
    out = torch.empty_like(gate) if out is None else out
    _check(_lib.uno_silu_mul(_ptr(gate), _ptr(up), _ptr(out), gate.numel(), _dtype_code(gate.dtype),
                             _stream(stream)))
    return out


def residual_add(a, b, out=None, stream=None):
    _need_cuda(a, b)
    out = torch.empty_like(a) if out is None else out
    _check(_lib.uno_residual_add(_ptr(a), _ptr(b), _ptr(out), a.numel(), _dtype_code(a.dtype), _stream(stream)))
    return out


def residual_rmsnorm(x, y, eps=1e-5, s_out=None, h_out=None, stream=None):
    """s = x + y and h = rmsnorm(s) in one launch; returns (s, h).  s_out may be x."""
    _need_cuda(x, y)
    M, K = x.shape
    s_out = torch.empty_like(x) if s_out is None else s_out
    h_out = torch.empty_like(x) if h_out is None else h_out
    _check(_lib.uno_residual_rmsnorm(_ptr(x), _ptr(y), _ptr(s_out), _ptr(h_out), M, K, float(eps),
                                     _dtype_code(x.dtype), _stream(stream)))
    return s_out, h_out


def header_symbols(header_path):
    """Names of the functions declared in include/uno.h (for ABI checks)."""
    text = open(header_path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(uno_[a-z0-9_]+)\s*\(", text)))

