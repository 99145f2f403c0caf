"""Build libuno.so (HIP for gfx950) in-tree with hipcc.

    python lossless_speculative_drafting_amd/build.py [--jobs N] [--verbose]

(run as a script: importing the package first would load the library it rebuilds)

Every source under csrc/ is compiled to an object in _build/ and linked into
lossless_speculative_drafting_amd/libuno.so.  The measurement probes under
probes/ (stand-alone HIP programs, not part of the library) are built next to
their sources.  Packed-fp32 instructions are disabled for all device code.
"""

import argparse
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(REPO, "_build", "libuno")
LIB_PATH = os.path.join(PKG_DIR, "libuno.so")
PROBES = os.path.join(PKG_DIR, "probes")
ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    "-I", os.path.join(REPO, "include"),
]


def _hipcc():
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found; set HIPCC or install ROCm")
    return cand


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line only
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)
    return obj


def _build_probe(src, verbose):
    exe = os.path.splitext(src)[0]
    cmd = [_hipcc(), *[f for f in COMMON_FLAGS if f != "-fPIC"], src, "-o", exe]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
        raise RuntimeError(f"probe build failed: {src}\n" + "\n".join(noise))
    return exe


def build(jobs=None, verbose=False):
    """Compile every source and link libuno.so (and build the probes); returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    probes = sorted(os.path.join(PROBES, f) for f in os.listdir(PROBES) if f.endswith(".hip")) \
        if os.path.isdir(PROBES) else []
    jobs = jobs or min(8, len(srcs) + len(probes))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        probe_jobs = [ex.submit(_build_probe, p, verbose) for p in probes]
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
        for j in probe_jobs:
            j.result()
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed\n" + res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    main()
