"""Builds libgr_beam.so (HIP kernels for gfx950 + host engine) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = [os.path.join(PKG, "csrc", f) for f in ("gr_kernels.hip", "gr_prefill.hip", "gr_chain.hip", "gr_engine.cpp")]
OUT = os.path.join(PKG, "libgr_beam.so")

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=gfx950",
    # keep the compiler from emitting packed fp32 vector ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every source into OUT (always recompiles).  Returns the library path."""
    tmp = OUT + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           *SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, OUT)
    build_timed(verbose)
    build_rate_probe(verbose)
    return OUT


TIMED_OUT = os.path.join(PKG, "libgr_beam_timed.so")


def build_timed(verbose: bool = False) -> str:
    """The same library with the context-attention wave timeline compiled in (GR_WAVE_TIMES):
    a measurement build that `bench.py --wave-times` loads in a child process; the product
    library has none of it."""
    tmp = TIMED_OUT + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-DGR_WAVE_TIMES", "-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(PKG, "csrc"), *SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on the wave-timeline build ({res.returncode}):\n{out}")
    os.replace(tmp, TIMED_OUT)
    return TIMED_OUT


PROBE_SRC = os.path.join(PKG, "csrc", "rate_probe.hip")
PROBE_OUT = os.path.join(PKG, "rate_probe")


def build_rate_probe(verbose: bool = False) -> str:
    """The unit-rate probe (a stand-alone executable: MFMA, FMA and exp2 issue rates measured on
    the GPU, the ceilings that `bench.py --rate-probe` reports next to the published peaks)."""
    tmp = PROBE_OUT + ".tmp"
    flags = [f for f in HIP_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [hipcc(), *flags, PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on the rate probe ({res.returncode}):\n{out}")
    os.replace(tmp, PROBE_OUT)
    return PROBE_OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
