"""Summaries of rocprofv3 output for the profiles/ folder (host-side text processing).

    python -m lossless_speculative_drafting_amd.rocprof_summary stats KERNEL_STATS_CSV \\
        --title TITLE --command CMD [--top N] [--group NAME=SUBSTRING ...]
        Markdown table of a `--kernel-trace --stats` run, plus named groups of
        kernels with their combined time per launch of the group's first member.

    python -m lossless_speculative_drafting_amd.rocprof_summary copy-probe [--mib N]
        Run one plain device copy of N MiB (torch copy_ of a bf16 tensor): the
        known-size reference whose FETCH_SIZE / WRITE_SIZE calibrate the counters.

    python -m lossless_speculative_drafting_amd.rocprof_summary trace KERNEL_TRACE_CSV --match SUBSTRING ...
        Launches of a `--kernel-trace` run by kernel and grid (calls, average,
        median, min, max duration), in order of first launch.

    python -m lossless_speculative_drafting_amd.rocprof_summary counters CSV [CSV ...] \\
        --group NAME=SUBSTRING ... [--copy-fetch CSV --copy-write CSV --copy-mib N] [--cus N]
        Per-dispatch averages of every counter of `--pmc` runs by kernel group,
        with derived figures: scaled FETCH_SIZE / WRITE_SIZE bytes and their
        rate over the counter run's duration, the clock (GRBM_GUI_ACTIVE, which
        adds up the --xcds XCDs' busy cycles, per XCD over the duration), MFMA
        busy as a share of the SIMD cycles (over cycles x CUs x 4), bf16 MFMA
        flop (512 per MOP), L2 hit rate, LDS bank-conflict cycles.

    python -m lossless_speculative_drafting_amd.rocprof_summary traffic \\
        --fetch CSV --write CSV --copy-fetch CSV --copy-write CSV --copy-mib N \\
        --key NAME --launch SUBSTRING [--also SUBSTRING] --source FILE ...
        HBM bytes per launch of a kernel from two `--pmc` runs (FETCH_SIZE, then
        WRITE_SIZE; KiB per dispatch), each scaled by the factor that makes the
        copy probe's reading equal its known size.  A launch is one dispatch of
        a kernel whose name contains --launch; dispatches matching --also
        (a split-K reduction, say) are counted into the launch they follow.
        Prints JSON with the digest of the named sources, so that a reader can
        tell whether the numbers still describe the current code.
"""

import argparse
import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def source_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short(name, width=96):
    name = name.replace("uno::(anonymous namespace)::", "")
    cut = name.find("(")
    if cut > 0 and not name.startswith("void at::"):
        name = name[:cut]
    return name if len(name) <= width else name[:width - 3] + "..."


def stats(args):
    rows = list(csv.DictReader(open(args.csv)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    out = [f"# {args.title}", "", "Command (run from the repository root on one MI355X):", "", "```",
           args.command, "```", "", "| kernel | calls | avg us | total ms | % |", "|---|---:|---:|---:|---:|"]
    for r in rows[:args.top]:
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |")
    if args.group:
        out += ["", "| group | launches | total ms | avg us per launch |", "|---|---:|---:|---:|"]
        for spec in args.group:
            gname, _, subs = spec.partition("=")
            parts = subs.split("|")
            launches = sum(int(r["Calls"]) for r in rows if parts[0] in r["Name"])
            tot = sum(float(r["TotalDurationNs"]) for r in rows if any(p in r["Name"] for p in parts))
            if launches:
                out.append(f"| {gname} | {launches} | {tot / 1e6:.3f} | {tot / launches / 1e3:.2f} |")
    out += ["", f"All kernels: {total / 1e6:.3f} ms."]
    print("\n".join(out))


def copy_probe(args):
    import torch
    n = args.mib * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {args.mib} MiB", flush=True)


def _per_dispatch(path, counter):
    """[(dispatch id, kernel name, value)] in dispatch order for one counter."""
    acc = defaultdict(float)
    names = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        acc[d] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    return [(d, names[d], acc[d]) for d in sorted(acc)]


def _copy_kib(path, counter):
    vals = [v for _, n, v in _per_dispatch(path, counter) if "copy" in n.lower()]
    if not vals:
        raise SystemExit(f"no copy kernel with {counter} in {path}")
    return max(vals)


def _launch_kib(path, counter, launch, also):
    per_launch, cur = [], None
    for _, name, v in _per_dispatch(path, counter):
        if launch in name:
            if cur is not None:
                per_launch.append(cur)
            cur = v
        elif also and any(a in name for a in also) and cur is not None:
            cur += v
    if cur is not None:
        per_launch.append(cur)
    if not per_launch:
        raise SystemExit(f"no dispatch of {launch!r} in {path}")
    return sum(per_launch) / len(per_launch), len(per_launch)


def traffic(args):
    known = args.copy_mib * float(1 << 20)
    f_fac = known / (_copy_kib(args.copy_fetch, "FETCH_SIZE") * 1024.0)
    w_fac = known / (_copy_kib(args.copy_write, "WRITE_SIZE") * 1024.0)
    f_kib, n_f = _launch_kib(args.fetch, "FETCH_SIZE", args.launch, args.also)
    w_kib, n_w = _launch_kib(args.write, "WRITE_SIZE", args.launch, args.also)
    rec = {
        "source_digest": source_digest(args.source),
        "sources": args.source,
        "launch_kernel": args.launch,
        "counted_with_it": args.also,
        "launches": [n_f, n_w],
        "fetch_kib_per_launch_raw": round(f_kib, 1),
        "write_kib_per_launch_raw": round(w_kib, 1),
        "fetch_scale": round(f_fac, 4),
        "write_scale": round(w_fac, 4),
        "bytes_per_launch": round(f_kib * 1024.0 * f_fac + w_kib * 1024.0 * w_fac),
    }
    path = args.out
    data = {}
    if path and os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data[args.key] = rec
    text = json.dumps(data, indent=1, sort_keys=True)
    if path:
        with open(path, "w") as f:
            f.write(text + "\n")
    print(text)


def _dispatches(path):
    """{dispatch id: (kernel name, duration ns, {counter: value summed over its rows})}."""
    out = {}
    for r in csv.DictReader(open(path)):
        d = int(r["Dispatch_Id"])
        if d not in out:
            dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            out[d] = (r["Kernel_Name"], dur, defaultdict(float))
        out[d][2][r["Counter_Name"]] += float(r["Counter_Value"])
    return out


def counters(args):
    """Per-dispatch averages of every counter in one or more --pmc runs, by kernel group,
    with the derived figures the counters allow (see the table notes)."""
    scale = {}
    known = args.copy_mib * float(1 << 20)
    if args.copy_fetch:
        scale["FETCH_SIZE"] = known / (_copy_kib(args.copy_fetch, "FETCH_SIZE") * 1024.0)
    if args.copy_write:
        scale["WRITE_SIZE"] = known / (_copy_kib(args.copy_write, "WRITE_SIZE") * 1024.0)
    groups = [g.split("=", 1) for g in args.group]
    rows = []
    for path in args.csv:
        disp = _dispatches(path)
        for gname, sub in groups:
            sel = [v for v in disp.values() if sub in v[0]]
            if not sel:
                continue
            n = len(sel)
            dur_us = sum(v[1] for v in sel) / n / 1e3
            avg = defaultdict(float)
            for v in sel:
                for k, x in v[2].items():
                    avg[k] += x / n
            rows.append((gname, os.path.basename(os.path.dirname(path)) or path, n, dur_us, dict(avg)))
    cus = args.cus
    lines = [f"| group | run | dispatches | us per dispatch (counter run) | figures per dispatch |",
             "|---|---|---:|---:|---|"]
    for gname, run, n, dur_us, c in rows:
        figs = []
        for k in ("FETCH_SIZE", "WRITE_SIZE"):
            if k in c:
                b = c[k] * 1024.0 * scale.get(k, 1.0)
                figs.append(f"{k} {b / 1e6:.2f} MB{' (scaled)' if k in scale else ' (raw KiB x 1024)'}"
                            f" = {b / dur_us / 1e3:.0f} GB/s")
        gui = c.get("GRBM_GUI_ACTIVE")
        if gui:
            cyc = gui / args.xcds  # (the counter adds up the busy cycles of every XCD)
            figs.append(f"{cyc / (dur_us * 1e3) * 1e3:.0f} MHz (GPU-busy cycles per XCD over the duration)")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                figs.append(f"MFMA busy {100.0 * c['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * cus * 4):.1f}% of SIMD cycles")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c:
            fl = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
            figs.append(f"bf16 MFMA {fl / 1e9:.1f} GFLOP = {fl / dur_us / 1e6:.0f} TFLOP/s")
        if "TCC_HIT_sum" in c and "TCC_MISS_sum" in c:
            tot = c["TCC_HIT_sum"] + c["TCC_MISS_sum"]
            figs.append(f"L2 hit {100.0 * c['TCC_HIT_sum'] / max(tot, 1.0):.1f}%")
        if "SQ_LDS_BANK_CONFLICT" in c and "SQ_LDS_IDX_ACTIVE" in c:
            figs.append(f"LDS bank-conflict cycles {100.0 * c['SQ_LDS_BANK_CONFLICT'] / max(c['SQ_LDS_IDX_ACTIVE'], 1.0):.1f}% of LDS-active")
        raw = ", ".join(f"{k} {v:.4g}" for k, v in sorted(c.items()))
        lines.append(f"| {gname} | {run} | {n} | {dur_us:.2f} | {'; '.join(figs)}<br>raw: {raw} |")
    text = "\n".join(lines)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")
    print(text)


def trace(args):
    """Launches of a `--kernel-trace` run by kernel and grid: calls and duration
    statistics, for the kernels whose names contain one of the --match substrings."""
    groups = defaultdict(list)
    first = {}
    for r in csv.DictReader(open(args.csv)):
        name = r["Kernel_Name"]
        hit = next((m for m in args.match if m in name), None)
        if hit is None:
            continue
        key = (_short(name), int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]),
               int(r["Workgroup_Size_X"]))
        d = int(r["Dispatch_Id"])
        first[key] = min(first.get(key, d), d)
        groups[key].append((d, (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    lines = ["| kernel | grid (threads) | workgroup | calls | avg us | median us | min us | max us |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for key in sorted(groups, key=lambda k: first[k]):
        v = sorted(t for _, t in groups[key])
        lines.append(f"| `{key[0]}` | {key[1]} | {key[2]} | {len(v)} | {sum(v) / len(v):.2f} | "
                     f"{v[len(v) // 2]:.2f} | {v[0]:.2f} | {v[-1]:.2f} |")
        if args.calls:  # every call's duration, in launch order
            lines.append("|  | calls in order: " + " ".join(f"{t:.1f}" for _, t in sorted(groups[key])) + " |||||||")
    print("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--top", type=int, default=16)
    s.add_argument("--group", action="append", default=[])
    c = sub.add_parser("copy-probe")
    c.add_argument("--mib", type=int, default=1024)
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-mib", type=int, default=1024)
    t.add_argument("--key", required=True)
    t.add_argument("--launch", required=True)
    t.add_argument("--also", action="append", default=[])
    t.add_argument("--source", action="append", required=True)
    t.add_argument("--out", default=None)
    tr = sub.add_parser("trace")
    tr.add_argument("csv")
    tr.add_argument("--match", action="append", required=True)
    tr.add_argument("--calls", action="store_true", help="also list every call's duration in launch order")
    k = sub.add_parser("counters")
    k.add_argument("csv", nargs="+")
    k.add_argument("--group", action="append", required=True, help="NAME=SUBSTRING of the kernel name")
    k.add_argument("--copy-fetch", default=None)
    k.add_argument("--copy-write", default=None)
    k.add_argument("--copy-mib", type=int, default=1024)
    k.add_argument("--cus", type=int, default=256)
    k.add_argument("--xcds", type=int, default=8)
    k.add_argument("--out", default=None)
    args = ap.parse_args(argv)
    {"stats": stats, "copy-probe": copy_probe, "traffic": traffic, "counters": counters, "trace": trace}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
