"""Build libbc.so (the HIP library behind include/bc.h) for gfx950 with hipcc.

The library is built in-tree, next to this file, so that it travels with the
source tree.  Every source is compiled with packed fp32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbc.so")
BUILD = os.path.join(HERE, "_build")
# the instrumented variant: the same kernels plus per-phase clock reads
LIB_CLK = os.path.join(HERE, "libbc_clk.so")
BUILD_CLK = os.path.join(HERE, "_build_clk")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["bc_gemv.hip", "bc_gemv_batch.hip", "bc_attn.hip", "bc_kv.hip", "bc_snap.hip", "bc_masked.hip", "bc_batch.hip",
           "bc_layer.hip", "bc_clock.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-ffp-contract=fast", "-munsafe-fp-atomics"]


def build(verbose: bool = False, jobs: int = 4, phase_clocks: bool = False) -> str:
    """Builds libbc.so, or with phase_clocks the instrumented libbc_clk.so
    (-DBC_PHASE_CLOCKS: the kernels also read the shader clock at phase
    ends; a measurement build, loaded with BC_LIBRARY=libbc_clk.so)."""
    lib, bdir = (LIB_CLK, BUILD_CLK) if phase_clocks else (LIB, BUILD)
    flags = FLAGS + (["-DBC_PHASE_CLOCKS"] if phase_clocks else [])
    objs = []
    procs = []
    for src in SOURCES:
        os.makedirs(bdir, exist_ok=True)
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        cmd = [HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    while procs:
        _wait(procs.pop(0))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


def _wait(item):
    src, proc = item
    _, err = proc.communicate()
    lines = [ln for ln in (err or "").splitlines() if "packed-fp32-ops" not in ln]
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(lines))
    if lines:
        print("\n".join(lines), file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, phase_clocks="--phase-clocks" in sys.argv))
