"""Build libqb.so (HIP, gfx950) in-tree.

Each translation unit is compiled by hipcc in parallel; the pass-1 kernels are
split into one unit per expert count.  Flags: no fast-math, no FMA
contraction (-ffp-contract=off) so fp32 sums and differences round exactly as
written; packed-fp32 instructions disabled; fp32 subnormals kept (HIP
default on gfx950).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqb.so")
# the diagnostic streaming kernels (the measured HBM ceiling), a separate library
PROBE_LIB = os.path.join(PKG, "libstreamprobe.so")
ARCH = os.environ.get("QB_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-fno-fast-math", "-fvisibility=hidden", "-Wall", "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

EXPERTS = (16, 32, 64, 128, 256)


def _units():
    units = [(f"qb_pass1_e{e}.o", "qb_pass1.hip", [f"-DQB_P1_E={e}"]) for e in EXPERTS]
    for src in ("qb_radix.hip", "qb_select.hip", "qb_k3_lei.hip", "qb_router.hip", "qb_metrics.hip",
                "qb_shard.hip", "qb_api.hip"):
        units.append((src.replace(".hip", ".o"), src, []))
    return units


def _compile(unit, verbose, build_dir, defines):
    obj, src, extra = unit
    out = os.path.join(build_dir, obj)
    cmd = [HIPCC, *CFLAGS, *extra, *defines, "-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature and says so
    msg = "\n".join(l for l in (p.stdout + p.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "unknown target feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg)
    return out


def build(verbose: bool = False, jobs: int | None = None, defines=(), out: str | None = None) -> str:
    """Compile and link libqb.so.  `defines` (e.g. ["-DQB_RH_UNROLL=16"])
    override the kernels' tuning constants; `out` puts the library (and its
    objects) elsewhere, for comparing such variants."""
    lib = out or LIB
    build_dir = os.path.join(os.path.dirname(lib), "_build") if out else BUILD
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda u: _compile(u, verbose, build_dir, list(defines)), _units()))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    if not out:
        build_probe(verbose)
    return lib


def build_probe(verbose: bool = False) -> str:
    """Compile libstreamprobe.so (include/stream_probe.h)."""
    os.makedirs(BUILD, exist_ok=True)
    obj = _compile(("stream_probe.o", "stream_probe.hip", []), verbose, BUILD, [])
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
