"""Build libmoe.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m quantized_moe_expert_top_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")

SOURCES = ["api.cpp", "router.hip", "route.hip", "permute.hip", "w4a16.hip", "w4a8.hip",
           "w8a8.hip", "combine.hip", "telemetry.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-function",
    "-fvisibility=hidden",
    # packed fp32 instructions stay off (hand-written or compiler-generated)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE float32 division: the W8A8 quantization scale and codes depend on it
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libmoe needs ROCm's hipcc to build")


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    probes = [os.path.join(HERE, "probes", name) for name in ("stream_read", "mfma_peak")]
    for probe in probes:
        r = subprocess.run([hipcc(), "--offload-arch=gfx950", "-O3", "-Xclang", "-target-feature",
                            "-Xclang", "-packed-fp32-ops", probe + ".hip", "-o", probe],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"probe build failed:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {LIB} and {', '.join(probes)}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
