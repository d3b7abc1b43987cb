"""Build libmoe.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Every kernel's register use is read from the compiler's resource-usage
remarks; the build fails if any kernel spills to scratch memory (the GEMM
pipelines count their outstanding loads by hand, which a spill inside the
loop would silently break, and a spill costs the decode kernels their
bandwidth).

Usage: python -m quantized_moe_expert_top_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import re
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


_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]):\s*(\S+)")


def kernel_resources(remarks: str) -> dict:
    """{kernel: {"vgprs", "agprs", "scratch", "occupancy"}} from the text of
    hipcc's -Rpass-analysis=kernel-resource-usage remarks (device pass)."""
    out, cur = {}, None
    keys = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch",
            "Occupancy [waves/SIMD]": "occupancy"}
    for m in _REMARK.finditer(remarks):
        field, val = m.group(1), m.group(2)
        if field == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[keys[field]] = int(val)
    return out


def spilling(resources: dict) -> dict:
    """Kernels whose scratch use is above zero: {kernel: bytes per lane}."""
    return {k: v["scratch"] for k, v in resources.items() if v.get("scratch", 0) > 0}


def _compile(src: str):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj, kernel_resources(r.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        done = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in done]
    resources = {k: v for _, res in done for k, v in res.items()}
    if not resources:
        raise RuntimeError("no kernel resource-usage remarks found in hipcc's output")
    spills = spilling(resources)
    if spills:
        lines = "\n".join(f"  {v:5d} B/lane  {k}" for k, v in sorted(spills.items()))
        raise RuntimeError(f"{len(spills)} kernel(s) spill to scratch memory:\n{lines}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}: {len(resources)} kernels, none spilling to scratch")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
