"""A stack of gated-LoRA layers driven through the C ABI.

The pages add the diffusion (LoRA) pathway to every projection of every
transformer layer ("How It Works: The 'Uno' Architecture" and "Two Decoupled
Weight Sets" on the aifromscratch.in page) and say nothing about the rest of
the layer.  This module runs the plainest Llama-like chain with the
attention mixing left out, every projection a gated-LoRA call on the same
mixed batch of verify and draft rows:

    h = rmsnorm(x); q, k, v = P_q(h), P_k(h), P_v(h); x = x + P_o(q)
    h = rmsnorm(x); x = x + P_down(silu(P_gate(h)) * P_up(h))

All intermediates live in buffers allocated once.  The rows are planned
once (uno_segment_rows) and every projection reuses the plan.  Projections
that read the same input run as one grouped launch (q, k, v; gate, up): their
W_AR and lora_b rows are stacked once at construction, their A matrices too,
so one LoRA down-projection yields T for the whole group and one grouped
gated GEMM writes each projection to its own buffer.  A layer is then four
down-projections and four gated GEMMs.  With fused=True (the default) gate
and up run with silu(g) * u in the GEMM epilogue (uno_gated_gemm_swiglu,
weights interleaved once at construction), bitwise the unfused chain under
the same plan.  (The residual add is not fused into o and down: their tiles
run one per CU, where the epilogue's read of the residual is not hidden, and
the separate add + norm launch costs less.)  With grouped=False every
projection runs on its own.  After the first call a forward pass launches only library kernels on
the current stream.
"""

import ctypes

import torch

from . import _lib

PROJECTIONS = ("q", "k", "v", "o", "gate", "up", "down")


GROUPS = (("q", "k", "v"), ("gate", "up"))


def _stack_group(layer, names):
    """Stacked (w, lora_a, lora_b) of the named projections, and views of each one's slices."""
    w = torch.cat([layer[n][0] for n in names], 0)
    a = torch.cat([layer[n][1] for n in names], 0)
    b = torch.cat([layer[n][2] for n in names], 0)
    views, n0, j0 = {}, 0, 0
    for n in names:
        N, r = layer[n][0].shape[0], layer[n][1].shape[0]
        views[n] = (w[n0:n0 + N], a[j0:j0 + r], b[n0:n0 + N])
        n0, j0 = n0 + N, j0 + r
    return (w, a, b, [layer[n][0].shape[0] for n in names]), views


class GatedLoraStack:
    def __init__(self, layers, gate, scale=2.0, eps=1e-5, grouped=True, fused=True):
        """layers: list of dicts name -> (w [N,K], lora_a [r,K], lora_b [N,r]) bf16 CUDA tensors.
        gate: uint8 CUDA tensor [M] (1 = draft row).

        With grouped=True the q/k/v and gate/up weights are copied once into
        stacked tensors; self.layers then holds views of those copies (the
        caller may drop its own)."""
        self.grouped = bool(grouped)
        self.groups = []
        if self.grouped:
            new_layers = []
            for layer in layers:
                lay = dict(layer)
                gl = {}
                for names in GROUPS:
                    stacked, views = _stack_group(layer, names)
                    gl[names] = stacked
                    lay.update(views)
                new_layers.append(lay)
                self.groups.append(gl)
            layers = new_layers
        self.layers = layers
        self.fused = self.grouped and bool(fused)
        self.swiglu = []
        if self.fused:
            for li, layer in enumerate(layers):
                wg, _, bg = layer["gate"]
                wu, _, bu = layer["up"]
                w_p, b_p = _lib.swiglu_pack(wg, wu, bg, bu)
                self.swiglu.append((w_p, self.groups[li][GROUPS[1]][1], b_p))
        self.gate = gate
        self.scale = float(scale)
        self.eps = float(eps)
        M = gate.shape[0]
        dev = gate.device
        l0 = layers[0]
        hidden = l0["q"][0].shape[1]
        kv = l0["k"][0].shape[0]
        ffn = l0["gate"][0].shape[0]
        r = l0["q"][1].shape[0]
        bf = torch.bfloat16
        self.M, self.hidden, self.kv, self.ffn, self.r = M, hidden, kv, ffn, r
        self.Md = int(gate.to(torch.int64).sum().item())  # draft rows (one host sync, here)
        self.timer = None
        self.t_timer = None
        self.h = torch.empty((M, hidden), dtype=bf, device=dev)
        self.q = torch.empty((M, hidden), dtype=bf, device=dev)
        self.k = torch.empty((M, kv), dtype=bf, device=dev)
        self.v = torch.empty((M, kv), dtype=bf, device=dev)
        self.o = torch.empty((M, hidden), dtype=bf, device=dev)
        self.g = torch.empty((M, ffn), dtype=bf, device=dev)
        self.u = torch.empty((M, ffn), dtype=bf, device=dev)
        self.act = torch.empty((M, ffn), dtype=bf, device=dev)
        self.dn = torch.empty((M, hidden), dtype=bf, device=dev)
        self.x = torch.empty((M, hidden), dtype=bf, device=dev)
        lib = _lib.library()
        need = 0
        for name in PROJECTIONS:
            w = l0[name][0]
            N, K = w.shape
            need = max(need, int(lib.uno_lora_down_workspace_size(M, K, r)),
                       int(lib.uno_gated_gemm_workspace_size(M, N, K, r)))
        t_width = r
        if self.grouped:
            for names, (w, a, b, ns) in self.groups[0].items():
                K = w.shape[1]
                arr = (ctypes.c_int64 * len(ns))(*ns)
                need = max(need, int(lib.uno_lora_down_workspace_size(M, K, a.shape[0])),
                           int(lib.uno_gated_gemm_grouped_workspace_size(M, K, r, arr, len(ns))))
                t_width = max(t_width, a.shape[0])
        if self.fused:
            w_p, a_st, b_p = self.swiglu[0]
            need = max(need, int(lib.uno_gated_gemm_swiglu_workspace_size(M, w_p.shape[0] // 2, w_p.shape[1],
                                                                          b_p.shape[1])))
        self.ws = _lib.Workspace(dev)
        self.ws.get(need)
        self.t = torch.empty(_lib.lora_t_size(M, t_width) // 2, dtype=bf, device=dev)
        self.plan = None

    def _timed(self, K, N, launch, out_cols=None, t_cols=None):
        """Run one gated-GEMM launch; with a timer list set, bracket it with
        HIP events on the current stream and record its algorithmic flops
        (2 M K N for the product, 2 Md r N for the adapter extension) and
        bytes (W and B once, x and y once, the draft rows of T once; y is
        out_cols wide and T t_cols wide when given)."""
        if self.timer is None:
            launch()
            return
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        launch()
        e1.record()
        M, Md, r = self.M, self.Md, self.r
        out_cols = N if out_cols is None else out_cols
        t_cols = r if t_cols is None else t_cols
        flops = 2.0 * M * K * N + 2.0 * Md * r * N
        nbytes = 2.0 * (N * K + N * r + M * K + M * out_cols + Md * t_cols)
        self.timer.append((e0, e1, flops, nbytes))

    def _lora(self, inp, a):
        """T for the draft rows; with t_timer set, bracketed by HIP events on the
        current stream and recorded with its algorithmic flops (2 Md K r) and
        bytes (the draft rows of x, A, and T's rows up to the next multiple of 32)."""
        if self.t_timer is None:
            _lib.lora_down(inp, a, self.plan, self.scale, t=self.t, workspace=self.ws)
            return
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _lib.lora_down(inp, a, self.plan, self.scale, t=self.t, workspace=self.ws)
        e1.record()
        r, K = a.shape
        Md = self.Md
        Md_pad = (Md + 31) // 32 * 32
        self.t_timer.append((e0, e1, 2.0 * Md * K * r, 2.0 * (Md * K + r * K + Md_pad * r)))

    def _proj(self, layer, name, inp, out):
        w, a, b = layer[name]
        self._lora(inp, a)
        self._timed(w.shape[1], w.shape[0],
                    lambda: _lib.gated_gemm(inp, w, self.t, b, self.plan, out=out, workspace=self.ws))

    def _group(self, li, names, inp, outs):
        w, a, b, ns = self.groups[li][names]
        self._lora(inp, a)
        self._timed(w.shape[1], w.shape[0],
                    lambda: _lib.gated_gemm_grouped(inp, w, self.t, b, self.plan, ns, outs=outs,
                                                    workspace=self.ws))

    def _swiglu(self, li, inp):
        """act = silu(P_gate(inp)) * P_up(inp) in one launch."""
        w_p, a_st, b_p = self.swiglu[li]
        self._lora(inp, a_st)
        self._timed(w_p.shape[1], w_p.shape[0],
                    lambda: _lib.gated_gemm_swiglu(inp, w_p, self.t, b_p, self.plan, out=self.act,
                                                   workspace=self.ws),
                    out_cols=w_p.shape[0] // 2, t_cols=a_st.shape[0])

    def _projections(self, li, layer, items, trace_into):
        """items: [(name, input, output)] sharing one input when grouped."""
        if self.grouped and len(items) > 1:
            self._group(li, tuple(n for n, _, _ in items), items[0][1], [o for _, _, o in items])
        else:
            for name, inp, out in items:
                self._proj(layer, name, inp, out)
        if trace_into is not None:
            for name, inp, out in items:
                trace_into[name] = (inp.clone(), out.clone())

    def forward(self, x_in, trace_layer=None, trace=None):
        """Run every layer on x_in [M, hidden] (not modified); returns the final hidden state.

        If trace is a dict, the inputs and outputs of each projection of layer
        `trace_layer` are cloned into it as trace[name] = (input, output).
        """
        self.x.copy_(x_in)
        self.plan = _lib.RowPlan(self.gate) if self.plan is None else self.plan
        # (unfused layers: each residual add followed by a norm is one launch,
        # bitwise the two separate ones)
        _lib.rmsnorm(self.x, self.eps, out=self.h)
        last = len(self.layers) - 1
        for li, layer in enumerate(self.layers):
            rec = trace if (trace is not None and li == trace_layer) else None
            self._projections(li, layer, [("q", self.h, self.q), ("k", self.h, self.k), ("v", self.h, self.v)], rec)
            self._projections(li, layer, [("o", self.q, self.o)], rec)
            _lib.residual_rmsnorm(self.x, self.o, self.eps, s_out=self.x, h_out=self.h)
            if self.fused and rec is None:  # (a traced layer runs unfused: its g and u then exist)
                self._swiglu(li, self.h)
            else:
                self._projections(li, layer, [("gate", self.h, self.g), ("up", self.h, self.u)], rec)
                _lib.silu_mul(self.g, self.u, out=self.act)
            self._projections(li, layer, [("down", self.act, self.dn)], rec)
            if li < last:
                _lib.residual_rmsnorm(self.x, self.dn, self.eps, s_out=self.x, h_out=self.h)
            else:
                _lib.residual_add(self.x, self.dn, out=self.x)
        return self.x
