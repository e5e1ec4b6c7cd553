"""Build the gfx950 HIP library in-tree with hipcc.

    python -m expert_serving_amd.build

Every source under csrc/ is compiled for gfx950 only and linked into
expert_serving_amd/libmoe_mi355x.so.  Packed-fp32 instructions are disabled
for all device code; the routing source is also built without floating-point
contraction so its fixed operation sequences stay as written.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["moe_api.hip", "router.hip", "route.hip", "dispatch.hip", "gemm.hip", "combine.hip",
           "mxfp8.hip", "ep.hip"]
PEAKS_SRC = "peaks.hip"
PEAKS_BIN = os.path.join(HERE, "moe_peaks")
NO_CONTRACT = {"route.hip"}

COMMON = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
          "-Wno-unused-function", "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src in NO_CONTRACT:
        cmd.insert(1, "-ffp-contract=off")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    errs = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    # the ceiling microbenchmark (a standalone program)
    cmd = [HIPCC, *[c for c in COMMON if c != "-fPIC"], os.path.join(CSRC, PEAKS_SRC), "-o", PEAKS_BIN]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PEAKS_SRC}:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {LIB} and {PEAKS_BIN}")
    return LIB


if __name__ == "__main__":
    build()
