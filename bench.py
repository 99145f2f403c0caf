"""Benchmark one Uno draft+verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-extras]

A step is one pass of the whole hot path over one batch of synthetic input:
the gated-LoRA forward of the mixed batch through every projection of the
layer stack (with the layer glue), fresh Philox uniforms, and block
verification of every sequence's drafted block.  Inputs (weights, hidden
states, logits, drafted tokens) are resident in HBM before timing starts.

Default workload: 32 layers x 7 projections of an 8B-shaped model
(4096 -> 4096/1024/1024/4096 and 4096 -> 14336 -> 4096, rank-128 LoRA,
alpha 256), 32 sequences x [16 verify | 16 draft] rows, verification of a
16-token block per sequence over a 128256-token vocabulary (draft noise
sigma = 1, T = 1).  Weights are random-initialised bf16; data is synthetic.

Prints one JSON line: verified tokens/s (emitted tokens summed over the timed
steps / elapsed time), the roofline of the dominant kernel (the gated GEMM,
bf16 MFMA: algorithmic flops 2MKN + 2 Md r N per launch over its HIP-event
time, every launch of the timed steps), block verification's HBM rate, and
the oracle timed on the host cores on a bounded sample.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
SCALE = 2.0                   # alpha / r = 256 / 128
EARLY_CHUNK = 4  # positions per chunk of the early-exit verifier


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="stack32_b32", choices=["stack32_b32", "layer_b1", "layer_b64"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    # (profiling runs: skip the measurements that follow the timed region --
    # early-exit verifier, LM head, tree verification -- so that a kernel
    # trace holds the timed steps' kernels only)
    ap.add_argument("--no-extras", action="store_true")
    return ap.parse_args()


def pct(sorted_vals, q):
    """The q-th percentile of an ascending list (linear interpolation)."""
    if len(sorted_vals) == 1:
        return sorted_vals[0]
    pos = (len(sorted_vals) - 1) * q / 100.0
    i = int(pos)
    j = min(i + 1, len(sorted_vals) - 1)
    return sorted_vals[i] + (sorted_vals[j] - sorted_vals[i]) * (pos - i)


def verify_bytes(B, L, V, esz=2, redraws=None):
    """Algorithmic bytes of block verification: both logit arrays once, the redraw row pair
    of each sequence that redraws, tokens, uniforms and outputs."""
    redraws = B if redraws is None else redraws
    return 2.0 * B * L * V * esz + redraws * 2.0 * V * esz + B * L * 4 + B * (L + 1) * 4 + B * (L + 3) * 4


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "lossless_speculative_drafting_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel_key, digest):
    """HBM bytes per launch from the committed counter summary, if it was taken on this source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sharding is described in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import lossless_speculative_drafting_amd as uno
    from synthetic import WORKLOADS, gate_vector
    from synthetic import device as sdev

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = WORKLOADS[args.workload]
    B, L, V = wl.n_seq, wl.block, wl.vocab
    M = wl.rows
    Md = wl.n_seq * wl.draft_rows
    T = wl.temperatures[0]
    sigma = 1.0 if 1.0 in wl.draft_sigmas else wl.draft_sigmas[0]

    # ---------------- resident inputs
    layers = [sdev.layer_weights(wl.projections, wl.seed * 1000 + 100 * i) for i in range(wl.layers)]
    gate_np = gate_vector(wl.n_seq, wl.verify_rows, wl.draft_rows)
    gate = torch.from_numpy(gate_np).to(dev)
    stack = uno.GatedLoraStack(layers, gate, SCALE)
    del layers  # the stack holds its own (stacked) copies
    x0 = sdev.randn((M, wl.projections[0][1]), 1.0, wl.seed)
    z, d = sdev.verify_logits(B, L, V, wl.seed, kind=wl.logits, target_sigma=wl.target_sigma,
                              draft_sigma=sigma)
    drafts = uno.draft_sample(d, uno.philox_uniforms(0, 1, 0, B * L, device=dev), T)
    u = torch.empty(B * (L + 1), dtype=torch.float32, device=dev)
    total_steps = args.warmup + args.steps
    n_acc = torch.empty((total_steps, B), dtype=torch.int32, device=dev)
    out_tok = torch.empty((total_steps, B, L + 1), dtype=torch.int32, device=dev)
    n_emit = torch.empty((total_steps, B), dtype=torch.int32, device=dev)
    vws = uno.Workspace(dev)
    torch.cuda.synchronize()

    verify_events = []

    def step(i, timed):
        # Per-launch events cost the stream a few microseconds each (about
        # 0.2 ms over the 128 gated-GEMM launches of a step), so they bracket
        # the launches of one timed step -- the last -- rather than of all.
        stack.timer = gemm_events if (timed and i == total_steps - 1) else None
        stack.forward(x0)
        uno.philox_uniforms(0, 0, i * B * (L + 1), B * (L + 1), out=u)
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        uno.block_verify(z, d, drafts, u, T, False, outputs=(n_acc[i], out_tok[i], n_emit[i]), workspace=vws)
        if timed:
            e1.record()
            verify_events.append((e0, e1, i))

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    # The dominant kernel (the gated GEMM) and block verification are timed
    # per launch with HIP events recorded on the stream they run on, inside
    # the timed steps themselves (the GEMM in the last timed step).
    gemm_events = []
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.warmup, total_steps):
        step(i, True)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stack.timer = None
    gpu_ms = ev0.elapsed_time(ev1)
    elapsed = max(wall, gpu_ms / 1e3)
    tokens = int(n_emit[args.warmup:].sum().item())
    ms_per_step = elapsed * 1e3 / args.steps
    value = tokens / elapsed

    gemm_s = sum(ev[0].elapsed_time(ev[1]) for ev in gemm_events) / 1e3
    gemm_flop = sum(ev[2] for ev in gemm_events)
    gemm_bytes = sum(ev[3] for ev in gemm_events)
    n_gemm = len(gemm_events)
    # The bound follows the arithmetic intensity against the ridge point
    # (2.5 PFLOP/s / 8 TB/s = 312 flop/B): a handful of rows streams the
    # weights (HBM-bound), a batch of hundreds of rows is MFMA-bound.
    mfma_bound = gemm_flop / gemm_bytes >= PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3
    if mfma_bound:
        gemm_achieved, gemm_peak, gemm_unit = gemm_flop / gemm_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        gemm_achieved, gemm_peak, gemm_unit = gemm_bytes / gemm_s / 1e9, PEAK_HBM_GBS, "GB/s"
    digest = source_digest("gemm.hip")
    # (the counters were taken on the default workload's launches)
    traffic = committed_traffic("gated_gemm", digest) if args.workload == "stack32_b32" else None
    # Per projection launch of a layer (the stack's order: q|k|v, o, gate|up
    # with SwiGLU, down), over the 32 layers of the bracketed step: median and
    # p10 / p90 time, and the algorithmic rate at the median.
    per_launch = {}
    kinds = ("q|k|v", "o", "gate|up", "down")
    if n_gemm % len(kinds) == 0:
        for j, kind in enumerate(kinds):
            evs = gemm_events[j::len(kinds)]
            ts = sorted(ev[0].elapsed_time(ev[1]) * 1e3 for ev in evs)
            med = pct(ts, 50)
            per_launch[kind] = {"median_us": round(med, 2), "p10_us": round(pct(ts, 10), 2),
                                "p90_us": round(pct(ts, 90), 2),
                                "tflops_at_median": round(evs[0][2] / med / 1e6, 1)}

    verify_early, lm_head, tree = None, None, None
    if not args.no_extras:
        # The early-exit verifier on the last step's inputs (outside the timed
        # region): its time per call, the share of logit rows it streams, and a
        # check that its outputs are the one-pass verifier's.
        last = total_steps - 1
        uno.philox_uniforms(0, 0, last * B * (L + 1), B * (L + 1), out=u)
        e_out = (torch.empty_like(n_acc[0]), torch.empty_like(out_tok[0]), torch.empty_like(n_emit[0]))
        ews = uno.Workspace(dev)
        for _ in range(3):
            uno.block_verify(z, d, drafts, u, T, False, outputs=e_out, workspace=ews, early_chunk=EARLY_CHUNK)
        ee0, ee1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ee0.record()
        for _ in range(20):
            uno.block_verify(z, d, drafts, u, T, False, outputs=e_out, workspace=ews, early_chunk=EARLY_CHUNK)
        ee1.record()
        torch.cuda.synchronize()
        same = all(torch.equal(a, b) for a, b in zip(e_out, (n_acc[last], out_tok[last], n_emit[last])))
        chunks_read = torch.clamp((n_acc[last].long() + EARLY_CHUNK) // EARLY_CHUNK, max=(L + EARLY_CHUNK - 1) // EARLY_CHUNK)
        rows_read = torch.clamp(chunks_read * EARLY_CHUNK, max=L).sum().item() / (B * L)
        verify_early = {"chunk": EARLY_CHUNK, "us_per_call": round(ee0.elapsed_time(ee1) / 20 * 1e3, 3),
                        "rows_read_frac": round(rows_read, 4), "same_outputs_as_one_pass": bool(same)}

        lm_head = lm_head_measure(uno, sdev, torch, B, L, V, wl.projections[0][1], T, wl.seed, dev)
        tree = tree_measure(uno, sdev, torch, B, V, T, wl.seed, dev)

    vt = sum(a.elapsed_time(b) for a, b, _ in verify_events) / 1e3 / len(verify_events)
    v_us = sorted(a.elapsed_time(b) * 1e3 for a, b, _ in verify_events)
    redraws = sum(int((n_acc[i] < L).sum().item()) for _, _, i in verify_events) / len(verify_events)
    v_gbs = verify_bytes(B, L, V, 2, redraws) / vt / 1e9

    result = {
        "metric": "verified tokens/s per draft+verify step",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init bf16 weights and logits)",
        "config": {
            "workload": f"{args.workload}: {wl.layers} layers x {len(wl.projections)} gated-LoRA projections "
                        f"(8B shapes, r=128, alpha=256), {wl.n_seq} seqs x [{wl.verify_rows} verify | "
                        f"{wl.draft_rows} draft] rows, verify block {L} over V={V}, sigma={sigma}, T={T}",
            "rows": M,
            "draft_rows": Md,
            "sequences": B,
            "block": L,
            "vocab": V,
            "tokens_per_step": round(tokens / args.steps, 3),
        },
        "roofline": {
            "bound": "mfma" if mfma_bound else "hbm",
            "kernel": "gated GEMM (gated_gemm_kernel, main mode, with its split-K reduction where planned): "
                      "every launch of the last timed step",
            "achieved": round(gemm_achieved, 2),
            "peak": gemm_peak,
            "unit": gemm_unit,
            "frac": round(gemm_achieved / gemm_peak, 4),
            "traffic": traffic,
            "launches": n_gemm,
            "avg_launch_us": round(gemm_s / n_gemm * 1e6, 3),
            "algorithmic_gflop_per_launch": round(gemm_flop / n_gemm / 1e9, 4),
            "algorithmic_mb_per_launch": round(gemm_bytes / n_gemm / 1e6, 3),
            "per_launch": per_launch,
        },
        "verify_roofline": {
            "bound": "hbm",
            "achieved": round(v_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(v_gbs / PEAK_HBM_GBS, 4),
            "us_per_call": round(vt * 1e6, 3),
            "median_us": round(pct(v_us, 50), 2),
            "p10_us": round(pct(v_us, 10), 2),
            "p90_us": round(pct(v_us, 90), 2),
            "redraws_per_call": redraws,
            "early_exit": verify_early,
        },
        "lm_head": lm_head,
        "tree_verify": tree,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, stack.layers, x0, z, d, drafts, u, gate_np, T, L)
    print(json.dumps(result), flush=True)


def lm_head_measure(uno, sdev, torch, B, L, V, K, T, seed, dev, reps=5):
    """The LM head fused with the verification statistics, on this workload's
    rows (B sequences x L drafted positions, target and draft rows: 2 B L rows
    of K = hidden over V tokens), outside the timed region.  Per-call times
    (HIP events, `reps` calls) of uno_lm_head_verify with the redraw rows
    recomputed (no logit row written) and with the logits stored, and of the
    unfused chain: the plain GEMM writing the logits, then uno_block_verify.
    Drafts come from the draft rows' own distribution.  All three must give
    the same outputs (up to the unfused verifier's different chunking of the
    statistics, which can move a decision only on an exact tie)."""
    bf = torch.bfloat16
    hidden, w, x, u = sdev.lm_head_tensors(B, L, V, K, seed + 501, kind="normal", device=dev)
    rows = hidden.shape[0]
    logits = torch.empty((rows, V), dtype=bf, device=dev)
    ws = uno.Workspace(dev)
    uno.lm_head_verify(hidden, w, x, u, T, logits=logits, workspace=ws)
    x = uno.draft_sample(logits[B * L:].view(B, L, V), uno.philox_uniforms(0, 7, 0, B * L, device=dev), T)
    plan = uno.RowPlan(torch.zeros(rows, dtype=torch.uint8, device=dev))  # every row an AR row: no adapter
    t0 = torch.zeros(uno.lora_t_size(rows, 8) // 2, dtype=bf, device=dev)
    b0 = torch.zeros((V, 8), dtype=bf, device=dev)
    gws, vws = uno.Workspace(dev), uno.Workspace(dev)

    def outs():
        return (torch.empty(B, dtype=torch.int32, device=dev), torch.empty((B, L + 1), dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev))

    def unfused(o):
        uno.gated_gemm(hidden, w, t0, b0, plan, out=logits, workspace=gws)
        uno.block_verify(logits[:B * L].view(B, L, V), logits[B * L:].view(B, L, V), x, u, T, False, outputs=o,
                         workspace=vws)

    calls = {
        "fused_recompute": lambda o: uno.lm_head_verify(hidden, w, x, u, T, outputs=o, workspace=ws),
        "fused_store": lambda o: uno.lm_head_verify(hidden, w, x, u, T, logits=logits, outputs=o, workspace=ws),
        "unfused": unfused,
    }
    res, got = {}, {}
    for name, fn in calls.items():
        o = outs()
        for _ in range(2):
            fn(o)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn(o)
        e1.record()
        torch.cuda.synchronize()
        res[name + "_us"] = round(e0.elapsed_time(e1) / reps * 1e3, 2)
        got[name] = o
    same = all(torch.equal(a, b) for a, b in zip(got["fused_recompute"], got["fused_store"]))
    agree = sum(int(torch.equal(got["fused_store"][1][s], got["unfused"][1][s])) for s in range(B)) / B
    flop = 2.0 * rows * V * K
    res.update({
        "rows": rows, "vocab": V, "hidden": K,
        "gemm_gflop": round(flop / 1e9, 2),
        "fused_store_tflops": round(flop / (res["fused_store_us"] * 1e-6) / 1e12, 1),
        "logit_bytes_not_written_mb": round(rows * V * 2 / 1e6, 1),
        "fused_modes_same_outputs": bool(same),
        "seqs_same_as_unfused_frac": round(agree, 4),
        "mean_accepted": round(float(got["fused_store"][0].float().mean().item()), 3),
    })
    return res


def tree_measure(uno, sdev, torch, B, V, T, seed, dev, K=2, D=5, reps=10):
    """Tree verification (the tree sampler) outside the timed region: B
    trees, each the K-ary prefix tree of depth D over per-depth top-K
    candidates (2^(D+1) - 1 = 63 nodes for K = 2, D = 5), node logits the
    depth's base logits plus noise, bf16 over V.  Per-call HIP-event time,
    and the rows the walks read (n_accepted + 1 per tree, each twice:
    statistics, then segment masses) per second."""
    N = (K ** (D + 1) - 1) // (K - 1) if K > 1 else D + 1
    parents, depth, frontier = [-1], [0], [0]
    for d in range(D):
        nxt = []
        for v in frontier:
            for _ in range(K):
                parents.append(v)
                depth.append(d + 1)
                nxt.append(len(parents) - 1)
        frontier = nxt
    base = sdev.randn((B, D + 1, V), 3.0, seed + 701, device=dev, dtype=torch.float32)
    dep = torch.tensor(depth, device=dev)
    z = (base[:, dep, :] + sdev.randn((B, N, V), 0.7, seed + 702, device=dev, dtype=torch.float32)).to(torch.bfloat16)
    top = torch.topk(base, K, dim=-1).indices  # [B, D + 1, K]: the candidates of each depth
    child_rank = torch.tensor([0] + [(i - 1) % K for i in range(1, N)], device=dev)
    parent_depth = torch.tensor([0] + [depth[i] - 1 for i in range(1, N)], device=dev)
    tokens = top[:, parent_depth, child_rank].to(torch.int32).contiguous()
    tokens[:, 0] = 0
    par = torch.tensor(parents, dtype=torch.int32, device=dev).expand(B, N).contiguous()
    u = uno.philox_uniforms(0, 9, 0, B * N, device=dev).view(B, N)
    ws = uno.Workspace(dev)
    out = uno.tree_verify(z.contiguous(), par, tokens, u, T, workspace=ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        uno.tree_verify(z, par, tokens, u, T, outputs=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    rows = float((out[0].float() + 1).sum())
    nbytes = 2.0 * rows * V * 2
    return {"trees": B, "nodes_per_tree": N, "branching": K, "depth": D, "vocab": V, "us_per_call": round(us, 2),
            "rows_read_per_tree": round(rows / B, 3), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "mean_accepted": round(float(out[0].float().mean()), 3)}


def cpu_baseline(wl, layers, x0, z, d, drafts, u, gate_np, T, L):
    """The fp64 oracle on the host cores: one layer of the stack and verification of a few sequences,
    scaled to a full step (layers x layer time + sequences x per-sequence verify time)."""
    import numpy as np

    import oracle
    from oracle import stack as ost

    cores = len(os.sched_getaffinity(0))
    h = lambda t: t.float().cpu().numpy()  # noqa: E731
    lw = {n: tuple(h(t) for t in layers[0][n]) for n, _, _ in wl.projections}
    x = h(x0)
    t0 = time.perf_counter()
    hn = ost.rmsnorm(x)
    q = oracle.gated_lora(hn, *lw["q"], gate_np, SCALE)
    oracle.gated_lora(hn, *lw["k"], gate_np, SCALE)
    oracle.gated_lora(hn, *lw["v"], gate_np, SCALE)
    x1 = ost.residual_add(x, oracle.gated_lora(q, *lw["o"], gate_np, SCALE))
    hn = ost.rmsnorm(x1)
    act = ost.silu_mul(oracle.gated_lora(hn, *lw["gate"], gate_np, SCALE),
                       oracle.gated_lora(hn, *lw["up"], gate_np, SCALE))
    ost.residual_add(x1, oracle.gated_lora(act, *lw["down"], gate_np, SCALE))
    layer_s = time.perf_counter() - t0
    n_seq = 4
    zz, dd = h(z[:n_seq]), h(d[:n_seq])
    uu = u.cpu().numpy().astype(np.float64).reshape(-1, L + 1)[:n_seq]
    t0 = time.perf_counter()
    res = oracle.block_verify(zz, dd, drafts[:n_seq].cpu().numpy(), uu, T, False)
    verify_s = time.perf_counter() - t0
    B = wl.n_seq
    step_s = wl.layers * layer_s + B / n_seq * verify_s
    tokens = float(res["n_emitted"].sum()) * B / n_seq
    return {
        "value": round(tokens / step_s, 4),
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"one of {wl.layers} layers (7 fp64 gated-LoRA projections + glue, {layer_s:.2f} s) and "
                   f"verification of {n_seq} of {B} sequences ({verify_s:.2f} s), scaled to one step "
                   f"({step_s:.1f} s); numpy BLAS on {cores} cores"),
    }


if __name__ == "__main__":
    main()
