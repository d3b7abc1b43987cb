"""Kernel-trace summary of a bench.py timed region, from a rocprofv3 database.

bench.py --mark wraps each timed region in a roctx range ("timed_steps
<workload>", "timed_ffn <workload>"). Taken with
`rocprofv3 --kernel-trace --marker-trace`, the trace then keeps those ranges,
and this script counts only the dispatches that start inside one of them: the
timed graph replays, without the eager pass, the warmup, the spread passes or
the separately timed rows. It prints a markdown table (calls, average and
total duration per kernel) and the per-step kernel sum beside the region's own
length per step.

    python trace_summary.py RESULTS.db "timed_steps decode_t2" --steps 20
"""
from __future__ import annotations

import argparse
import json
import re
import sqlite3
from collections import defaultdict


def short_name(name: str) -> str:
    n = name.replace("moe::(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*", "", n)


def region(db, label: str):
    """(start, end) in ns of the roctx range whose message is `label`."""
    for start, end, extdata in db.execute("select start, end, extdata from regions"):
        try:
            msg = json.loads(extdata or "{}").get("message")
        except ValueError:
            msg = None
        if msg == label:
            return start, end
    raise SystemExit(f"no roctx range named {label!r} in the trace")


def summarize(path: str, label: str, steps: int) -> dict:
    db = sqlite3.connect(path)
    r0, r1 = region(db, label)
    per = defaultdict(list)
    for name, start, dur in db.execute("select name, start, duration from kernels"):
        if r0 <= start <= r1:
            per[short_name(name)].append(dur)
    rows = sorted(((n, len(d), sum(d) / len(d), sum(d)) for n, d in per.items()),
                  key=lambda r: -r[3])
    total = sum(r[3] for r in rows)
    return {"label": label, "region_ns": r1 - r0, "steps": steps, "rows": rows,
            "kernel_ns": total}


def markdown(s: dict) -> str:
    out = ["| kernel | calls | avg (us) | total (us) | share |", "|---|---:|---:|---:|---:|"]
    for n, c, avg, tot in s["rows"]:
        out.append(f"| `{n}` | {c} | {avg / 1e3:.2f} | {tot / 1e3:.1f} | "
                   f"{100.0 * tot / s['kernel_ns']:.1f}% |")
    st = s["steps"]
    out.append("")
    out.append(f"Kernel time inside the range: {s['kernel_ns'] / 1e3:.1f} us over {st} steps = "
               f"{s['kernel_ns'] / 1e3 / st:.2f} us per step; the range itself lasted "
               f"{s['region_ns'] / 1e3:.1f} us = {s['region_ns'] / 1e3 / st:.2f} us per step "
               f"(launch gaps and the host's event records make up the difference).")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db")
    ap.add_argument("label")
    ap.add_argument("--steps", type=int, required=True,
                    help="steps (or FFN passes) the timed range covers")
    a = ap.parse_args()
    print(markdown(summarize(a.db, a.label, a.steps)))


if __name__ == "__main__":
    main()
