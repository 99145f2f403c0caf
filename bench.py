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
EARLY_CHUNK = 6  # positions in the early-exit verifier's first chunk (then 12, 24, ...)


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
    # (the per-workload measurements of the other configurations: skipped,
    # or only one of them -- profiling runs)
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--only-config", default=None, choices=["tiny", "layer_b1", "layer_b64", "serve_b256"])
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
        print("bench.py measures one GPU only: the library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import lossless_speculative_drafting_amd as uno
    from synthetic import WORKLOADS, gate_vector
    from synthetic import device as sdev

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only_config:
        print(json.dumps({args.only_config: CONFIG_MEASURES[args.only_config](uno, sdev, torch, dev)}), flush=True)
        return
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
    z_sample, d_sample = z[:8].clone(), d[:8].clone()  # the oracle baseline's sequences
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

    # The LoRA down-projections (the launch and its split-K reduction) of one
    # more forward pass, outside the timed region: per-launch HIP events, the
    # algorithmic rate against the bf16 peak and their share of a step.
    lora_events = []
    stack.t_timer = lora_events
    stack.forward(x0)
    stack.t_timer = None
    torch.cuda.synchronize()
    lora_s = sum(ev[0].elapsed_time(ev[1]) for ev in lora_events) / 1e3
    lora_flop = sum(ev[2] for ev in lora_events)
    lora_bytes = sum(ev[3] for ev in lora_events)
    lora_kinds = {}
    if len(lora_events) % len(kinds) == 0:
        for j, kind in enumerate(kinds):
            evs = lora_events[j::len(kinds)]
            ts = sorted(ev[0].elapsed_time(ev[1]) * 1e3 for ev in evs)
            lora_kinds[kind] = {"median_us": round(pct(ts, 50), 2), "gflop": round(evs[0][2] / 1e9, 3),
                                "mb": round(evs[0][3] / 1e6, 2)}
    lora_roofline = {
        "bound": "latency",
        "kernel": "LoRA down-projection (T-mode tile and its split-K reduction, or the weight-streaming kernel) "
                  "of every projection group of one forward pass",
        "launches": len(lora_events),
        "avg_launch_us": round(lora_s / max(len(lora_events), 1) * 1e6, 3),
        "per_step_ms": round(lora_s * 1e3, 3),
        "share_of_step": round(lora_s * 1e3 / ms_per_step, 4),
        "achieved_tflops": round(lora_flop / lora_s / 1e12, 2) if lora_s > 0 else None,
        "frac_of_bf16_peak": round(lora_flop / lora_s / 1e12 / PEAK_BF16_TFLOPS, 4) if lora_s > 0 else None,
        "achieved_gbs": round(lora_bytes / lora_s / 1e9, 1) if lora_s > 0 else None,
        "traffic": committed_traffic("lora_down", digest) if args.workload == "stack32_b32" else None,
        "per_launch": lora_kinds,
    }

    # Block verification per call with its logits cold (outside the timed
    # region): back-to-back calls over three logit sets -- the step's and two
    # more of the same recipe, 0.79 GB, three times the 256 MB MALL -- with
    # one event pair around them, so that neither the MALL nor the few
    # microseconds an event pair costs enter a call's time.  The early-exit
    # verifier is timed the same way, with its share of the logit rows
    # streamed and a check that its outputs are the one-pass verifier's.
    last = total_steps - 1
    uno.philox_uniforms(0, 0, last * B * (L + 1), B * (L + 1), out=u)  # the last step's uniforms
    vsets = [(z, d, drafts)]
    for c in (1, 2):
        zc, dc = sdev.verify_logits(B, L, V, wl.seed + 7919 * c, kind=wl.logits, target_sigma=wl.target_sigma,
                                    draft_sigma=sigma)
        vsets.append((zc, dc, uno.draft_sample(dc, uno.philox_uniforms(0, 1, c * B * L, B * L, device=dev), T)))

    def verify_cold(chunk, n=21):
        outs = [(torch.empty_like(n_acc[0]), torch.empty_like(out_tok[0]), torch.empty_like(n_emit[0]))
                for _ in vsets]
        for i in range(len(vsets)):
            zz, dd, xx = vsets[i]
            uno.block_verify(zz, dd, xx, u, T, False, outputs=outs[i], workspace=vws, early_chunk=chunk)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for i in range(n):
            zz, dd, xx = vsets[i % len(vsets)]
            uno.block_verify(zz, dd, xx, u, T, False, outputs=outs[i % len(vsets)], workspace=vws,
                             early_chunk=chunk)
        c1.record()
        torch.cuda.synchronize()
        return c0.elapsed_time(c1) * 1e3 / n, outs

    v_cold_us, v_outs = verify_cold(None)
    cold_redraws = sum(int((o[0] < L).sum().item()) for o in v_outs) / len(v_outs)

    verify_early, lm_head, tree = None, None, None
    if not args.no_extras:
        early_us, e_outs = verify_cold(EARLY_CHUNK)
        same = all(torch.equal(a, b) for oe, ov in zip(e_outs, v_outs) for a, b in zip(oe, ov))
        # rows streamed: up to the end of the chunk (lengths EARLY_CHUNK, 2 EARLY_CHUNK, ...)
        # holding the first rejection
        ends, e, ln = [], 0, EARLY_CHUNK
        while e < L:
            e = min(L, e + ln)
            ends.append(e)
            ln *= 2
        na = [a for o in v_outs for a in o[0].cpu().tolist()]
        rows_read = sum(next(x for x in ends if x > min(a, L - 1)) for a in na) / (len(na) * L)
        verify_early = {"chunk": EARLY_CHUNK, "us_per_call": round(early_us, 3),
                        "rows_read_frac": round(rows_read, 4), "same_outputs_as_one_pass": bool(same)}

        lm_head = lm_head_measure(uno, sdev, torch, B, L, V, wl.projections[0][1], T, wl.seed, dev)
        tree = tree_measure(uno, sdev, torch, B, V, T, wl.seed, dev)

    platform = platform_info(torch)  # (right after the timed steps: clocks under recent load)
    configs = None
    if not args.no_configs:
        del z, d, vsets, v_outs
        torch.cuda.empty_cache()
        configs = {name: fn(uno, sdev, torch, dev) for name, fn in CONFIG_MEASURES.items()}

    # in the timed steps: per-call events (each pair adds a few microseconds)
    v_us = sorted(a.elapsed_time(b) * 1e3 for a, b, _ in verify_events)
    v_gbs = verify_bytes(B, L, V, 2, cold_redraws) / (v_cold_us * 1e-6) / 1e9

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
        "lora_down_roofline": lora_roofline,
        "verify_roofline": {
            "bound": "hbm",
            "achieved": round(v_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(v_gbs / PEAK_HBM_GBS, 4),
            "us_per_call": round(v_cold_us, 3),
            "timing": "back-to-back calls over three logit sets (0.79 GB, MALL defeated), one event pair",
            "redraws_per_call": cold_redraws,
            "in_step_event_us": {"median": round(pct(v_us, 50), 2), "p10": round(pct(v_us, 10), 2),
                                 "p90": round(pct(v_us, 90), 2)},
            "early_exit": verify_early,
        },
        "lm_head": lm_head,
        "tree_verify": tree,
        "configs": configs,
        "platform": platform,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, stack.layers, x0, z_sample, d_sample, drafts, u, gate_np, T, L)
    print(json.dumps(result), flush=True)


def lm_head_measure(uno, sdev, torch, B, L, V, K, T, seed, dev, reps=7):
    """The LM head fused with the verification statistics, on this workload's
    rows (B sequences x L drafted positions, target and draft rows: 2 B L rows
    of K = hidden over V tokens), outside the timed region.  Median per-call
    times (HIP events, `reps` calls each, the forms interleaved) of
    uno_lm_head_verify with the redraw rows recomputed (no logit row written)
    and with the logits stored, and of the unfused chain: the plain GEMM
    writing the logits, then uno_block_verify.
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
    # The three forms interleaved call by call (the order rotating each
    # round), each call between its own events: the clock drifts over a
    # second of back-to-back 1 ms GEMMs, and timing the forms one after
    # another would hand that drift to whichever form ran last.
    res, got, times = {}, {name: outs() for name in calls}, {name: [] for name in calls}
    names = list(calls)
    for r in range(2 + reps):
        for j in range(len(names)):
            name = names[(r + j) % len(names)]
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            calls[name](got[name])
            e1.record()
            if r >= 2:
                times[name].append((e0, e1))
    torch.cuda.synchronize()
    for name in names:
        ts = sorted(a.elapsed_time(b) * 1e3 for a, b in times[name])
        res[name + "_us"] = round(ts[len(ts) // 2], 2)
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


def platform_info(torch):
    """What the numbers were measured on: device, ROCm and torch versions, and the
    clocks, power and performance level rocm-smi reports (None where unavailable)."""
    import subprocess

    props = torch.cuda.get_device_properties(0)
    info = {"gpu": props.name, "arch": getattr(props, "gcnArchName", None), "cus": props.multi_processor_count,
            "torch": torch.__version__, "torch_hip": torch.version.hip, "rocm": None, "smi": None}
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        pass
    if "rocprof" in os.environ.get("LD_PRELOAD", ""):
        # (under the profiler the tool's library is preloaded into every child;
        # rocm-smi's launcher would replace itself in a process that has it)
        info["smi"] = "not queried under the profiler"
        return info
    try:
        out = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--showmaxpower", "--showperflevel",
                              "--json"], capture_output=True, text=True, timeout=30)
        cards = json.loads(out.stdout)
        card = next(iter(v for k, v in cards.items() if k.startswith("card")), None)
        if card:
            keep = ("sclk", "mclk", "fclk", "socclk", "power", "perf")
            info["smi"] = {k.strip(" :"): v for k, v in card.items() if any(w in k.lower() for w in keep)}
    except Exception as e:  # noqa: BLE001  (metadata only: never fail the bench on it)
        info["smi"] = f"unavailable: {type(e).__name__}"
    return info


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _median(xs):
    return pct(sorted(xs), 50)


def _layer_gemm_measure(uno, sdev, torch, wl, dev, copies=3, reps=6):
    """One 8B-shaped layer (seven gated-LoRA projections as four launches:
    grouped q|k|v, o, gate|up with SwiGLU, down) over the workload's mixed
    batch, rotating through `copies` independent copies of the weights so that
    a repetition never finds its weights in the 256 MB MALL (each forward
    touches about 320 MB of weights; a copy is reused only after the others'
    640 MB).  Per launch kind: median time of the gated GEMM (HIP events) and
    its algorithmic rate; the whole layer (LoRA down-projections and glue
    included) per repetition, timed in a forward pass of its own without the
    per-launch events."""
    from synthetic import gate_vector

    gate = torch.from_numpy(gate_vector(wl.n_seq, wl.verify_rows, wl.draft_rows)).to(dev)
    stacks = [uno.GatedLoraStack([sdev.layer_weights(wl.projections, wl.seed * 1000 + 7919 * c)], gate, SCALE)
              for c in range(copies)]
    x0 = sdev.randn((wl.rows, wl.projections[0][1]), 1.0, wl.seed + 3)
    for st in stacks:
        st.forward(x0)
    torch.cuda.synchronize()
    kinds = ("q|k|v", "o", "gate|up", "down")
    per = {k: [] for k in kinds}
    layer_us = []
    for i in range(reps * copies):
        st = stacks[(2 * i) % copies]
        # the whole layer without per-launch events (each event pair costs the
        # stream a few microseconds), then the same layer on the next copy of
        # the weights with an event pair around each gated GEMM (the copies
        # are used in turn, each again only after the other two)
        a, b = _events(torch)
        # (the GPU spins while the host enqueues the layer, so that the events
        # time the kernels and not the host's launch rate)
        torch.cuda._sleep(1_000_000)
        a.record()
        st.forward(x0)
        b.record()
        torch.cuda.synchronize()
        layer_us.append(a.elapsed_time(b) * 1e3)
        st = stacks[(2 * i + 1) % copies]
        st.timer = []
        torch.cuda._sleep(1_000_000)
        st.forward(x0)
        torch.cuda.synchronize()
        for k, ev in zip(kinds, st.timer):
            per[k].append((ev[0].elapsed_time(ev[1]) * 1e3, ev[2], ev[3]))
        st.timer = None
    out, tot_f, tot_b, tot_t = {}, 0.0, 0.0, 0.0
    for k in kinds:
        t = _median([p[0] for p in per[k]])
        f, nb = per[k][0][1], per[k][0][2]
        tot_f, tot_b, tot_t = tot_f + f, tot_b + nb, tot_t + t
        out[k] = {"median_us": round(t, 2), "tflops": round(f / t / 1e6, 1), "gbs": round(nb / t / 1e3, 1)}
    del stacks
    torch.cuda.empty_cache()
    return out, {"gemm_us": round(tot_t, 2), "gflop": round(tot_f / 1e9, 2), "mb": round(tot_b / 1e6, 1),
                 "tflops": round(tot_f / tot_t / 1e6, 1), "gbs": round(tot_b / tot_t / 1e3, 1),
                 "layer_us_median": round(_median(layer_us), 2)}


def _verify_measure(uno, sdev, torch, B, L, V, seed, kind, sigma, temps, dev, copies=1, reps=10, zipf_slope=1.1):
    """Block verification per call: `reps` calls back to back between one
    event pair (after two warm-up calls), each with its own uniforms and
    output buffers, rotating through `copies` independent logit sets so that
    the sets together exceed the MALL.  Drafts are drawn on the GPU from each
    set's draft logits at the call's temperature.  Per temperature: mean time
    per call, algorithmic GB/s (with the redraws that happened) and the
    tokens emitted per call."""
    sets = [sdev.verify_logits(B, L, V, seed + 13 * c, kind=kind, target_sigma=3.0, draft_sigma=sigma,
                               zipf_slope=zipf_slope) for c in range(copies)]
    res = {}
    ws = uno.Workspace(dev)
    n = reps + 2
    outs = [(torch.empty(B, dtype=torch.int32, device=dev), torch.empty((B, L + 1), dtype=torch.int32, device=dev),
             torch.empty(B, dtype=torch.int32, device=dev)) for _ in range(n)]
    u = uno.philox_uniforms(0, 0, 0, n * B * (L + 1), device=dev).view(n, B * (L + 1))
    for T in temps:
        drafts = [uno.draft_sample(d, uno.philox_uniforms(0, 1, 0, B * L, device=dev), T) for _, d in sets]

        def call(i):
            z, d = sets[i % copies]
            uno.block_verify(z, d, drafts[i % copies], u[i], T, False, outputs=outs[i], workspace=ws)

        for i in range(2):
            call(i)
        a, b = _events(torch)
        torch.cuda._sleep(200_000)  # (the host enqueues the calls while the GPU spins)
        a.record()
        for i in range(2, n):
            call(i)
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b) * 1e3 / reps
        emitted = sum(int(outs[i][2].sum().item()) for i in range(2, n))
        redraws = sum(int((outs[i][0] < L).sum().item()) for i in range(2, n))
        nbytes = verify_bytes(B, L, V, 2, redraws / reps)
        res[f"T={T}"] = {"us_per_call": round(t, 2), "gbs": round(nbytes / t / 1e3, 1),
                         "frac": round(nbytes / t / 1e3 / PEAK_HBM_GBS, 4),
                         "tokens_per_call": round(emitted / reps, 2),
                         "verify_only_tokens_per_s": round(emitted / reps / (t * 1e-6), 1)}
    del sets
    torch.cuda.empty_cache()
    return res


def measure_tiny(uno, sdev, torch, dev, reps=10):
    """The small fp32 configuration: one 512 -> 512 gated-LoRA projection over
    2 sequences x [8 verify | 4 draft] rows, and block verification of 10**6
    trials of one block (L = 4, V = 64, fp32 logits broadcast with sequence
    stride 0: the same block for every trial, as in the lossless chi-square
    test).  Both are latency-bound; reported as time per call, trials and
    verified tokens per second, and the mean emitted length beside its
    closed form (sum over m < L of the product of the first m acceptance
    rates, sum min(p, q) per position)."""
    import numpy as np

    from synthetic import WORKLOADS, gate_vector, gemm_inputs, verify_inputs

    wl = WORKLOADS["tiny"]
    L, V, T = wl.block, wl.vocab, 1.0
    trials = int(wl.extra["trials"])
    gate = gate_vector(wl.n_seq, wl.verify_rows, wl.draft_rows)
    (_, K, N), = wl.projections
    inp = gemm_inputs(gate.size, K, N, 128, seed=wl.seed, dtype="f32", gate=gate)
    x, w, a, b = (torch.from_numpy(np.ascontiguousarray(inp[k], dtype=np.float32)).to(dev) for k in ("x", "w", "a", "b"))
    g = torch.from_numpy(gate).to(dev)
    ws = uno.Workspace(dev)
    y = uno.gated_lora_fwd(x, w, a, b, g, SCALE, workspace=ws)
    tg = []
    for _ in range(reps):
        e0, e1 = _events(torch)
        torch.cuda._sleep(200_000)
        e0.record()
        uno.gated_lora_fwd(x, w, a, b, g, SCALE, out=y, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        tg.append(e0.elapsed_time(e1) * 1e3)
    z, d = verify_inputs(1, L, V, wl.seed, "normal", wl.target_sigma, wl.draft_sigmas[0], dtype="f32")
    zt, dt = (torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(dev) for v in (z, d))
    xd = uno.draft_sample(dt, uno.philox_uniforms(0, 1, 0, trials * L, device=dev), T, B=trials, L=L, V=V,
                          seq_stride=0)
    u = uno.philox_uniforms(0, 0, 0, trials * (L + 1), device=dev)
    vws = uno.Workspace(dev)
    outs = (torch.empty(trials, dtype=torch.int32, device=dev), torch.empty((trials, L + 1), dtype=torch.int32, device=dev),
            torch.empty(trials, dtype=torch.int32, device=dev))
    call = lambda: uno.block_verify(zt, dt, xd, u, T, False, B=trials, L=L, V=V, target_seq_stride=0,  # noqa: E731
                                    draft_seq_stride=0, outputs=outs, workspace=vws)
    call()
    tv = []
    for _ in range(reps):
        e0, e1 = _events(torch)
        torch.cuda._sleep(200_000)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        tv.append(e0.elapsed_time(e1) * 1e3)
    t_v = _median(tv)
    emitted = int(outs[2].sum().item())
    zz, dd = z[0].astype(np.float64), d[0].astype(np.float64)
    p = np.exp(zz - zz.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    q = np.exp(dd - dd.max(axis=1, keepdims=True))
    q /= q.sum(axis=1, keepdims=True)
    alpha = np.minimum(p, q).sum(axis=1)
    expect = float(sum(np.prod(alpha[:m]) for m in range(L)))
    return {"workload": "one 512->512 fp32 gated-LoRA projection over 2 seqs x [8 verify | 4 draft] rows; verify "
                        "10^6 trials of one block (L=4, V=64, fp32, sequence stride 0), T=1",
            "gemm": {"us_per_call": round(_median(tg), 2)},
            "verify": {"us_per_call": round(t_v, 2), "trials_per_s": round(trials / (t_v * 1e-6), 1),
                       "verified_tokens_per_s": round(emitted / (t_v * 1e-6), 1),
                       "mean_emitted": round(emitted / trials, 5), "mean_emitted_closed_form": round(expect, 5)}}


def measure_layer_b1(uno, sdev, torch, dev):
    """Batch 1 (one sequence of [16 verify | 16 draft] rows): the layer's
    gated GEMMs stream their weights (HBM-bound, ~31 flop/B), verification
    of 16 positions over V = 128256 is latency (8.2 MB; 64 logit sets are
    rotated so each call reads from HBM, not the MALL)."""
    from synthetic import WORKLOADS

    wl = WORKLOADS["layer_b1"]
    kinds, layer = _layer_gemm_measure(uno, sdev, torch, wl, dev)
    layer["bound"], layer["frac"] = "hbm", round(layer["gbs"] / PEAK_HBM_GBS, 4)
    ver = _verify_measure(uno, sdev, torch, wl.n_seq, wl.block, wl.vocab, wl.seed, "normal", 1.0, (1.0,), dev,
                          copies=64, reps=20)
    return {"workload": "1 layer x 7 projections, 1 seq x [16 verify | 16 draft] rows; verify 1 x 16 over "
                        "V=128256, sigma=1, T=1; weights rotated over 3 copies, logits over 64 (MALL defeated)",
            "gemm_per_launch": kinds, "gemm_layer": layer, "verify": ver}


def measure_layer_b64(uno, sdev, torch, dev):
    """Batch 64 (64 sequences x [16 | 16] rows, M = 2048): the layer's gated
    GEMMs are MFMA-bound; verification of 1024 positions (525 MB of logits)
    at draft noise sigma 0.25, 1 and 4."""
    from synthetic import WORKLOADS

    wl = WORKLOADS["layer_b64"]
    kinds, layer = _layer_gemm_measure(uno, sdev, torch, wl, dev)
    layer["bound"], layer["frac"] = "mfma", round(layer["tflops"] / PEAK_BF16_TFLOPS, 4)
    ver = {}
    for sigma in wl.draft_sigmas:
        ver[f"sigma={sigma}"] = _verify_measure(uno, sdev, torch, wl.n_seq, wl.block, wl.vocab, wl.seed, "normal",
                                                sigma, (1.0,), dev, copies=2)["T=1.0"]
    return {"workload": "1 layer x 7 projections, 64 seqs x [16 verify | 16 draft] rows (M=2048); verify "
                        "64 x 16 over V=128256, sigma in {0.25, 1, 4}, T=1; weights rotated over 3 copies, logits over 2",
            "gemm_per_launch": kinds, "gemm_layer": layer, "verify": ver}


def measure_serve_b256(uno, sdev, torch, dev, reps=4):
    """Large-batch serving (256 sequences x [32 | 32] rows, M = 16384): the
    up (4096 -> 14336) and down (14336 -> 4096) gated-LoRA projections,
    MFMA-bound, each as its LoRA down-projection plus its gated GEMM; then
    verification of 8192 positions over V = 128256 with Zipf-skewed logits
    (4.2 GB) at T = 0.6 and 1.0."""
    from synthetic import WORKLOADS, gate_vector

    wl = WORKLOADS["serve_b256"]
    M = wl.rows
    Md = wl.n_seq * wl.draft_rows
    gate = torch.from_numpy(gate_vector(wl.n_seq, wl.verify_rows, wl.draft_rows)).to(dev)
    plan = uno.RowPlan(gate)
    gemm = {}
    ws = uno.Workspace(dev)
    for i, (name, K, N) in enumerate(wl.projections):
        w, a, b = sdev.projection_weights(K, N, wl.seed * 1000 + 10 * i)
        x = sdev.randn((M, K), 1.0, wl.seed + i)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        t = uno.lora_down(x, a, plan, SCALE, workspace=ws)
        uno.gated_gemm(x, w, t, b, plan, out=y, workspace=ws)
        tg, tl = [], []
        for _ in range(reps):
            e0, e1 = _events(torch)
            e2, e3 = _events(torch)
            torch.cuda._sleep(200_000)  # (the host enqueues both launches while the GPU spins)
            e0.record()
            uno.lora_down(x, a, plan, SCALE, t=t, workspace=ws)
            e1.record()
            e2.record()
            uno.gated_gemm(x, w, t, b, plan, out=y, workspace=ws)
            e3.record()
            torch.cuda.synchronize()
            tl.append(e0.elapsed_time(e1) * 1e3)
            tg.append(e2.elapsed_time(e3) * 1e3)
        t_g, t_l = _median(tg), _median(tl)
        flop = 2.0 * M * K * N + 2.0 * Md * 128 * N
        flop_l = 2.0 * Md * K * 128
        gemm[name] = {"gemm_us": round(t_g, 2), "gemm_tflops": round(flop / t_g / 1e6, 1),
                      "gemm_frac": round(flop / t_g / 1e6 / PEAK_BF16_TFLOPS, 4),
                      "lora_down_us": round(t_l, 2),
                      "projection_tflops": round((flop + flop_l) / (t_g + t_l) / 1e6, 1)}
        del w, a, b, x, y, t
        torch.cuda.empty_cache()
    ver = _verify_measure(uno, sdev, torch, wl.n_seq, wl.block, wl.vocab, wl.seed, "zipf", wl.draft_sigmas[0],
                          wl.temperatures, dev, reps=5, zipf_slope=wl.extra["zipf_slope"])
    return {"workload": "up 4096->14336 and down 14336->4096 gated-LoRA projections (r=128), 256 seqs x "
                        "[32 verify | 32 draft] rows (M=16384); verify 256 x 32 over V=128256, Zipf logits "
                        "(slope 1.1, noise 0.5), T in {0.6, 1.0}",
            "gemm": gemm, "verify": ver}


CONFIG_MEASURES = {"tiny": measure_tiny, "layer_b1": measure_layer_b1, "layer_b64": measure_layer_b64, "serve_b256": measure_serve_b256}


def cpu_baseline(wl, layers, x0, z, d, drafts, u, gate_np, T, L, budget_s=10.0):
    """The fp64 oracle on the host cores: the stack's layers in order (each
    layer's weights brought to the host before its clock starts) until about
    `budget_s` seconds of compute, and verification of the sequences given,
    scaled to a full step (layers x mean layer time + sequences x
    per-sequence verify time)."""
    import numpy as np

    import oracle
    from oracle import stack as ost

    cores = len(os.sched_getaffinity(0))
    h = lambda t: t.float().cpu().numpy()  # noqa: E731
    x = h(x0)
    layer_s, n_layers = 0.0, 0
    for li in range(wl.layers):
        lw = {n: tuple(h(t) for t in layers[li][n]) for n, _, _ in wl.projections}
        t0 = time.perf_counter()
        hn = ost.rmsnorm(x)
        q = oracle.gated_lora(hn, *lw["q"], gate_np, SCALE)
        oracle.gated_lora(hn, *lw["k"], gate_np, SCALE)
        oracle.gated_lora(hn, *lw["v"], gate_np, SCALE)
        x1 = ost.residual_add(x, oracle.gated_lora(q, *lw["o"], gate_np, SCALE))
        hn = ost.rmsnorm(x1)
        act = ost.silu_mul(oracle.gated_lora(hn, *lw["gate"], gate_np, SCALE),
                           oracle.gated_lora(hn, *lw["up"], gate_np, SCALE))
        x = ost.residual_add(x1, oracle.gated_lora(act, *lw["down"], gate_np, SCALE))
        layer_s += time.perf_counter() - t0
        n_layers += 1
        del lw
        if layer_s >= budget_s:
            break
    n_seq = z.shape[0]
    zz, dd = h(z), h(d)
    uu = u.cpu().numpy().astype(np.float64).reshape(-1, L + 1)[:n_seq]
    t0 = time.perf_counter()
    res = oracle.block_verify(zz, dd, drafts[:n_seq].cpu().numpy(), uu, T, False)
    verify_s = time.perf_counter() - t0
    B = wl.n_seq
    step_s = wl.layers * layer_s / n_layers + B / n_seq * verify_s
    tokens = float(res["n_emitted"].sum()) * B / n_seq
    return {
        "value": round(tokens / step_s, 4),
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{n_layers} of {wl.layers} layers in order (7 fp64 gated-LoRA projections + glue each, "
                   f"{layer_s:.2f} s) and verification of {n_seq} of {B} sequences ({verify_s:.2f} s), scaled "
                   f"to one step ({step_s:.1f} s); numpy BLAS on {cores} cores"),
    }


if __name__ == "__main__":
    main()
