"""HBM traffic per launch of the dominant unit, from rocprofv3 counters.

Two counter passes per workload (FETCH_SIZE, then WRITE_SIZE; each reports
KiB per dispatch) are scaled by what the same counter reports for a plain
copy of known size (probes/stream_read copy: 262144 KiB read and written per
dispatch), then summed over the kernels one launch of the unit dispatches.
The result is stored with a hash of the kernel sources it was measured on;
bench.py reports it only while that hash still matches.

    python traffic.py --workload decode_t2 \\
        --calib-fetch C1.csv --calib-write C2.csv --fetch F.csv --write W.csv
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "quantized_moe_expert_top_amd", "csrc")
STORE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_KIB = 262144.0

# kernels one launch of the dominant unit (the unit bench.py times for the
# workload's default path) dispatches, by workload
_LAYER = [r"route_topk", r"permute_", r"w4a16_", r"decode_", r"combine_kernel"]
UNIT_KERNELS = {
    "decode_t2": ("moe_layer_w4a16", _LAYER),
    "decode_large": ("moe_layer_w4a16", _LAYER),
    "prefill_t512": ("moe_layer_w4a16", _LAYER),
    "w4a8_t512": ("moe_grouped_w4a8_ffn", [r"quant_rows_kernel", r"w4a8_mfma_kernel"]),
    "w8a8_t4096": ("moe_grouped_w8a8_ffn",
                   [r"act_quant_kernel", r"w8a8_mfma_kernel", r"h_quant_kernel"]),
}


def source_hash() -> str:
    """Hash of every kernel source the library is built from."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def kernel_means(path: str) -> dict:
    """{kernel name: (dispatches, mean counter value)} of one counter CSV."""
    acc = defaultdict(list)
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            acc[row["Kernel_Name"]].append(float(row["Counter_Value"]))
    return {k: (len(v), sum(v) / len(v)) for k, v in acc.items()}


def copy_factor(path: str) -> float:
    """Counter KiB reported per KiB actually moved by the copy dispatches."""
    means = kernel_means(path)
    hits = [m for k, (n, m) in means.items() if re.search(r"_Z2cpP|^cp\(", k)]
    if not hits:
        raise SystemExit(f"{path}: no copy-kernel dispatches")
    return hits[0] / COPY_KIB


def unit_kib(path: str, patterns) -> tuple:
    """Sum over the unit's kernels of their mean KiB per dispatch."""
    means = kernel_means(path)
    total, names = 0.0, []
    for name, (n, m) in sorted(means.items()):
        if any(re.search(p, name) for p in patterns):
            total += m
            short = re.sub(r"^void ", "", name).replace("moe::(anonymous namespace)::", "")
            names.append(re.sub(r"\(.*", "", short))
    return total, names


def lookup(workload: str):
    """Stored bytes per launch for this workload, or None if absent or stale."""
    try:
        with open(STORE) as f:
            entry = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not entry or entry.get("source_sha256") != source_hash():
        return None
    return entry


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True, choices=sorted(UNIT_KERNELS))
    ap.add_argument("--calib-fetch", required=True)
    ap.add_argument("--calib-write", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--command", default="")
    a = ap.parse_args()
    unit, pats = UNIT_KERNELS[a.workload]
    ff, fw = copy_factor(a.calib_fetch), copy_factor(a.calib_write)
    fk, names = unit_kib(a.fetch, pats)
    wk, _ = unit_kib(a.write, pats)
    fetch_b = fk / ff * 1024.0
    write_b = wk / fw * 1024.0
    entry = {
        "unit": unit,
        "kernels": names,
        "fetch_bytes_per_launch": int(fetch_b),
        "write_bytes_per_launch": int(write_b),
        "bytes_per_launch": int(fetch_b + write_b),
        "fetch_factor": round(ff, 4),
        "write_factor": round(fw, 4),
        "command": a.command,
        "source_sha256": source_hash(),
    }
    store = {}
    if os.path.exists(STORE):
        with open(STORE) as f:
            store = json.load(f)
    store[a.workload] = entry
    os.makedirs(os.path.dirname(STORE), exist_ok=True)
    with open(STORE, "w") as f:
        json.dump(store, f, indent=1, sort_keys=True)
    print(json.dumps({a.workload: entry}, indent=1))


if __name__ == "__main__":
    main()
