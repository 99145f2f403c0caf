"""A stack of gated-LoRA layers driven through the C ABI.

The pages add the diffusion (LoRA) pathway to every projection of every
transformer layer ("How It Works: The 'Uno' Architecture" and "Two Decoupled
Weight Sets" on the aifromscratch.in page) and say nothing about the rest of
the layer.  This driver runs the plainest Llama-like chain with the
attention mixing left out, every projection a gated-LoRA call on the same
mixed batch of verify and draft rows:

    h = rmsnorm(x); q, k, v = P_q(h), P_k(h), P_v(h); x = x + P_o(q)
    h = rmsnorm(x); x = x + P_down(silu(P_gate(h)) * P_up(h))

All intermediates live in buffers allocated once.  The rows are planned
once (uno_segment_rows) and every projection reuses the plan: one LoRA
down-projection and one gated GEMM per projection.  After the first call a
forward pass launches only library kernels on the current stream.
"""

import torch

from . import _lib

PROJECTIONS = ("q", "k", "v", "o", "gate", "up", "down")


class GatedLoraStack:
    def __init__(self, layers, gate, scale=2.0, eps=1e-5):
        """layers: list of dicts name -> (w [N,K], lora_a [r,K], lora_b [N,r]) bf16 CUDA tensors.
        gate: uint8 CUDA tensor [M] (1 = draft row)."""
        self.layers = layers
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
        need = 0
        for name in PROJECTIONS:
            w = l0[name][0]
            N, K = w.shape
            need = max(need, int(_lib.library().uno_lora_down_workspace_size(M, K, r)),
                       int(_lib.library().uno_gated_gemm_workspace_size(M, N, K, r)))
        self.ws = _lib.Workspace(dev)
        self.ws.get(need)
        self.t = torch.empty(_lib.lora_t_size(M, r) // 2, dtype=bf, device=dev)
        self.plan = None

    def _proj(self, layer, name, inp, out):
        w, a, b = layer[name]
        _lib.lora_down(inp, a, self.plan, self.scale, t=self.t, workspace=self.ws)
        _lib.gated_gemm(inp, w, self.t, b, self.plan, out=out, workspace=self.ws)

    def forward(self, x_in, trace_layer=None, trace=None):
        """Run every layer on x_in [M, hidden] (not modified); returns the final hidden state.

        If trace is a dict, the inputs and outputs of each projection of layer
        `trace_layer` are cloned into it as trace[name] = (input, output).
        """
        self.x.copy_(x_in)
        self.plan = _lib.RowPlan(self.gate) if self.plan is None else self.plan
        for li, layer in enumerate(self.layers):
            rec = trace is not None and li == trace_layer
            _lib.rmsnorm(self.x, self.eps, out=self.h)
            for name, inp, out in (("q", self.h, self.q), ("k", self.h, self.k), ("v", self.h, self.v),
                                   ("o", self.q, self.o)):
                self._proj(layer, name, inp, out)
                if rec:
                    trace[name] = (inp.clone(), out.clone())
            _lib.residual_add(self.x, self.o, out=self.x)
            _lib.rmsnorm(self.x, self.eps, out=self.h)
            for name, inp, out in (("gate", self.h, self.g), ("up", self.h, self.u)):
                self._proj(layer, name, inp, out)
                if rec:
                    trace[name] = (inp.clone(), out.clone())
            _lib.silu_mul(self.g, self.u, out=self.act)
            self._proj(layer, "down", self.act, self.dn)
            if rec:
                trace["down"] = (self.act.clone(), self.dn.clone())
            _lib.residual_add(self.x, self.dn, out=self.x)
        return self.x
