"""Builds libqubo.so (HIP, gfx950) in-tree with hipcc.

    python -m ising_ground_state_amd.build

The library is the C-ABI of include/qubo.h: host planning (plan.cpp), the HIP
kernels (kernels.hip, kernels_f64.hip), the host side of the searches (host.hip,
run_int.hip, run_f64.hip, run_steps.hip) and the entry points (capi.hip, and
noalloc.hip for the search that allocates nothing).

The same call builds lib/qubo_valu_rate from csrc/valu_rate.hip: a stand-alone
program that measures the vector ALU's issue rate per instruction form, the
peak the search kernels are priced against.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libqubo.so")
SOURCES = ["plan.cpp", "kernels.hip", "kernels_f64.hip", "host.hip", "run_int.hip", "run_f64.hip", "run_steps.hip",
           "capi.hip", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
VALU_RATE_SOURCE = "valu_rate.hip"
VALU_RATE_PATH = os.path.join(LIB_DIR, "qubo_valu_rate")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    # never let the compiler form packed FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Leave wave-uniform branches unstructured (they run as scalar branches).
    # Structurizing the search kernel's uniform body-loop branches added flow
    # blocks whose undefined incoming values are VGPRs; the scalar threshold
    # and counters then moved to VGPRs with copies in every 32-step body.
    "-mllvm", "-structurizecfg-skip-uniform-regions",
    "-Wall",
]


def build(verbose: bool = False) -> str:
    """Compile every source into lib/libqubo.so (always recompiles)."""
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I" + INCLUDE, "-I" + CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libqubo.so")
    if verbose and res.stderr.strip():
        # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
        lines = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, LIB_PATH)
    build_valu_rate(verbose)
    return LIB_PATH


def build_valu_rate(verbose: bool = False) -> str:
    """Compile the issue-rate program into lib/qubo_valu_rate (always recompiles)."""
    tmp = VALU_RATE_PATH + ".tmp%d" % os.getpid()
    flags = [f for f in FLAGS if f not in ("-shared", "-fPIC", "-fvisibility=hidden")]
    cmd = [HIPCC, *flags, os.path.join(CSRC, VALU_RATE_SOURCE), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building qubo_valu_rate")
    os.replace(tmp, VALU_RATE_PATH)
    return VALU_RATE_PATH


if __name__ == "__main__":
    print(build(verbose=True))
