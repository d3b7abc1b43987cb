"""Build the measurement probes (streaming-read / copy ceiling, MFMA-only
ceiling) for gfx950, in place next to their sources.

    python probes/build.py
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PROBES = ("stream_read", "mfma_peak")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> list:
    outs = []
    for name in PROBES:
        src, out = os.path.join(HERE, name + ".hip"), os.path.join(HERE, name)
        r = subprocess.run([hipcc(), "--offload-arch=gfx950", "-O3", "-Xclang", "-target-feature",
                            "-Xclang", "-packed-fp32-ops", src, "-o", out],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"probe build failed ({name}):\n{r.stdout}\n{r.stderr}")
        outs.append(out)
    if verbose:
        print("built " + ", ".join(outs))
    return outs


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
