"""Builds libsynth_gen.so (device generator of the seeded bf16 inputs) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "synth_gen.hip")
OUT = os.path.join(HERE, "libsynth_gen.so")


def build(verbose: bool = False) -> str:
    """Compile SRC into OUT (always recompiles).  Returns the library path."""
    from semantic_id_beam_amd.build import HIP_FLAGS, hipcc
    tmp = OUT + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
