"""Benchmark of the routed MoE FFN layer on one MI355X.

A step is one pass of the whole path (route -> permute -> grouped FFN ->
combine) over one batch. Default workload: decode of two concurrent requests,
T=2, H=2048, I=768, E=128, k=8, W4A16 g128, 48 independent layers per step
(so one step is one decode step through a 48-layer MoE stack). All inputs are
seeded synthetic tensors resident in HBM before the timed region.

Prints one JSON line with the whole-job throughput (tokens/s) of the chosen
workload, a roofline entry for its dominant unit, and the CPU oracle's
throughput on a bounded sample of the same workload. The default run also
carries a `prefill` block measured in the same process on the prompt
workload (T=4096, W8A8 on int8 MFMA): grouped-FFN time per layer, its int8
MFMA fraction, its HBM fraction and its measured traffic.

Algorithmic bytes per unit (the roofline's numerator) are what the method
must move: the packed weights and scales of the experts the unit routes to,
x in, the router logits in and out in. Intermediates (h, the grouped y) are
overheads of the design and show up only in the measured traffic.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_PEAK = {"bf16": 2500.0, "int8": 5000.0}   # dense, TFLOP/s (TOP/s for int8)
# streaming-read ceiling measured on one MI355X with probes/stream_read (plain
# 16-byte loads, 402.7 MB per kernel): the achievable side of the HBM roofline
HBM_MEASURED_CEILING_GBS = 6320.0
METRIC = "MoE-FFN tokens/s; decode HBM GB/s % of peak; prefill MFMA % of peak"
PREFILL_WORKLOAD = "w8a8_t4096"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_t2", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prompt-workload block of the default run")
    ap.add_argument("--eager", action="store_true", help="launch from Python instead of HIP graphs")
    ap.add_argument("--path", choices=("layer", "calls"), default=None,
                    help="layer: moe_layer_w4a16 (one call per layer; W4A16 only); "
                         "calls: the four separate calls. Default: layer for W4A16")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    ap.add_argument("--units", type=int, default=None,
                    help="stage only the first N units (short counter passes; per-launch "
                         "figures do not depend on the number of units)")
    ap.add_argument("--mark", action="store_true",
                    help="wrap each timed region in a roctx range (for kernel traces)")
    return ap.parse_args()


class Marker:
    """roctx ranges around timed regions (no-ops unless --mark and a roctx
    library loads); a kernel trace taken with --marker-trace can then keep
    only the dispatches inside them."""

    def __init__(self, on: bool):
        self.lib = None
        if on:
            for name in ("librocprofiler-sdk-roctx.so.1", "/opt/rocm/lib/librocprofiler-sdk-roctx.so.1",
                         "libroctx64.so", "/opt/rocm/lib/libroctx64.so"):
                try:
                    self.lib = ctypes.CDLL(name)
                    break
                except OSError:
                    continue

    def push(self, label: str):
        if self.lib is not None:
            self.lib.roctxRangePushA(label.encode())

    def pop(self):
        if self.lib is not None:
            self.lib.roctxRangePop()


def stage(wl, torch):
    """Upload every unit's inputs. Returns per-unit (x, logits, weights)."""
    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).cuda()

    units = []
    wcache = {}
    for u in range(wl.units):
        wu = 0 if wl.shared_weights else u
        if wu not in wcache:
            arrs = synth.layer_w8(wl, wu) if wl.fmt == "w8a8" else synth.layer_w4(wl, wu)
            wcache[wu] = tuple(dev(a) for a in arrs)
            del arrs
        units.append((dev(synth.x_bf16(wl, u)), dev(synth.router_logits(wl, u)), wcache[wu]))
    torch.cuda.synchronize()
    return units


def expert_bytes(wl) -> int:
    if wl.fmt in ("w4a16", "w4a8"):
        return (2 * wl.I * wl.H // 2 + 2 * wl.I * (wl.H // 128) * 2
                + wl.H * wl.I // 2 + wl.H * (wl.I // 128) * 2)
    return 2 * wl.I * wl.H + 2 * wl.I * 4 + wl.H * wl.I + wl.H * 4


def io_bytes(wl) -> int:
    """Layer I/O the method must move besides weights: x (bf16), router
    logits (float32) and out (float32)."""
    return wl.T * wl.H * 2 + wl.T * wl.E * 4 + wl.T * wl.H * 4


def layers_per_step(wl) -> list:
    """Units one step runs: every layer (decode/prefill stacks) or one unit."""
    if wl.name in ("decode_t2", "prefill_t512", "prefill_t512_flat"):
        return [list(range(wl.units))]
    return [[u] for u in range(wl.units)]


def measure(wl, args, torch, moe, marker, path=None):
    """Stage the workload, time K steps of the whole path (HIP graph per step
    unless --eager), then its dominant unit; returns the figures."""
    units = stage(wl, torch)
    bufs = [moe.LayerBuffers.alloc(wl.T, wl.H, wl.I, wl.E, wl.k, wl.fmt) for _ in range(wl.units)]
    shape = (wl.T, wl.H, wl.I, wl.E, wl.k)
    ffn = {"w4a16": moe.grouped_w4a16_ffn, "w4a8": moe.grouped_w4a8_ffn,
           "w8a8": moe.grouped_w8a8_ffn}[wl.fmt]
    schedule = layers_per_step(wl)

    def ffn_call(u):
        x, _, (w13, s13, w2, s2) = units[u]
        b = bufs[u]
        ffn(shape, x, w13, s13, w2, s2, b.offsets, b.sorted_slot, b.active, b.n_active, b.y,
            b.ffn_ws)

    path = path or ("layer" if wl.fmt == "w4a16" else "calls")
    if path == "layer" and wl.fmt != "w4a16":
        raise SystemExit("--path layer covers W4A16 workloads")

    def layer(u):
        x, L, wts = units[u]
        b = bufs[u]
        if path == "layer":
            moe.moe_layer(b, x, L, wts)
            return
        moe.route_topk(L, wl.k, b.ids, b.w)
        moe.permute(b.ids, wl.E, b.offsets, b.sorted_slot, b.slot_pos, b.active, b.n_active,
                    b.perm_ws)
        ffn_call(u)
        moe.combine(b.y, b.slot_pos, b.w, b.out)

    # one eager pass: checks the device once, leaves every unit's routing in place
    for u in range(wl.units):
        layer(u)
    torch.cuda.synchronize()
    act_per_unit = {u: int(bufs[u].n_active.cpu()[0]) for u in range(wl.units)}
    # routed rows per expert in each unit (the load the grouped kernels see)
    loads = np.stack([np.diff(bufs[u].offsets[:wl.E + 1].cpu().numpy()) for u in range(wl.units)])
    top = np.sort(loads, axis=1)[:, ::-1]
    expert_rows = {"mean_per_active_expert": round(float(loads.sum() / (loads > 0).sum()), 2),
                   "max_mean_over_units": round(float(top[:, 0].mean()), 2),
                   "max": int(top[:, 0].max()),
                   "top4_mean": round(float(top[:, :4].mean()), 2),
                   "active_experts_mean": round(float((loads > 0).sum(axis=1).mean()), 2)}

    # one HIP graph per step (the whole path for every layer of the step), and
    # one per step holding only the grouped-FFN calls (the dominant kernel)
    step_graphs, ffn_graphs = [], []
    if not args.eager:
        for us in schedule:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for u in us:
                    layer(u)
            step_graphs.append(g)
            if path == "calls":
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for u in us:
                        ffn_call(u)
                ffn_graphs.append(g)

    def run_step(i):
        if args.eager:
            for u in schedule[i % len(schedule)]:
                layer(u)
        else:
            step_graphs[i % len(schedule)].replay()

    def run_ffn(i):
        if args.eager:
            for u in schedule[i % len(schedule)]:
                ffn_call(u)
        else:
            ffn_graphs[i % len(schedule)].replay()

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        run_step(i)
        if path == "calls":
            run_ffn(i)
    torch.cuda.synchronize()

    # timed region: exactly K steps of the whole path
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    marker.push(f"timed_steps {wl.name}")
    t0.record(stream)
    wall0 = time.perf_counter()
    for i in range(args.steps):
        run_step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    marker.pop()
    ms_total = t0.elapsed_time(t1)
    ms_per_step = ms_total / args.steps

    # spread: three more passes of K steps each, after the timed region
    pass_ms = []
    for _ in range(3):
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for i in range(args.steps):
            run_step(i)
        a1.record(stream)
        torch.cuda.synchronize()
        pass_ms.append(a0.elapsed_time(a1) / args.steps)
    spread = {"passes_ms_per_step": [round(x, 4) for x in pass_ms],
              "median_ms_per_step": round(float(np.median(pass_ms)), 4)}

    # cold-cache steps (large-expert decode): a 1 GiB write between steps,
    # outside the timed window, evicts the 256 MB MALL before each step
    cold_ms = None
    if wl.name == "decode_large" and not args.eager:
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        cold = []
        for i in range(len(schedule)):
            scratch.zero_()
            c0 = torch.cuda.Event(enable_timing=True)
            c1 = torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            run_step(i)
            c1.record(stream)
            torch.cuda.synchronize()
            cold.append(c0.elapsed_time(c1))
        del scratch
        cold_ms = float(np.median(cold))
        spread["cold_median_ms_per_step"] = round(cold_ms, 4)
        spread["warm_ms_per_step"] = round(ms_per_step, 4)

    calls = [u for i in range(args.steps) for u in schedule[i % len(schedule)]]
    if path == "layer":
        # dominant unit: the whole-layer call (its kernels carry all of the
        # layer's bytes); per-call time from the timed region itself
        avg_ms = ms_total / len(calls)
        kernel = ("moe_layer_w4a16 (whole layer: fused decode gate/up + down kernels)"
                  if wl.T <= 4 else
                  "moe_layer_w4a16 (whole layer: route, permute, grouped MFMA FFN, combine)")
    else:
        # dominant unit: the grouped FFN calls of the same K steps, back to
        # back on the same stream, timed with HIP events
        f0 = torch.cuda.Event(enable_timing=True)
        f1 = torch.cuda.Event(enable_timing=True)
        marker.push(f"timed_ffn {wl.name}")
        f0.record(stream)
        for i in range(args.steps):
            run_ffn(i)
        f1.record(stream)
        torch.cuda.synchronize()
        marker.pop()
        avg_ms = f0.elapsed_time(f1) / len(calls)
        kernel = f"moe_grouped_{wl.fmt}_ffn (gate/up + down kernels)"
    eb = expert_bytes(wl)
    avg_bytes = sum(act_per_unit[u] * eb + io_bytes(wl) for u in calls) / len(calls)
    flops_per_call = 6.0 * wl.H * wl.I * wl.T * wl.k
    return {
        "wl": wl, "path": path, "schedule": schedule, "units": units, "bufs": bufs,
        "ms_total": ms_total, "ms_per_step": ms_per_step, "wall": wall, "spread": spread,
        "cold_ms": cold_ms, "avg_ms": avg_ms, "avg_bytes": avg_bytes, "kernel": kernel,
        "flops_per_call": flops_per_call,
        "mean_active": float(np.mean(list(act_per_unit.values()))),
        "expert_rows": expert_rows,
        "time_launches": lambda fn, n=50: time_launches(fn, args, torch, stream, n),
    }


def time_launches(fn, args, torch, stream, n=50):
    """Average device time of fn() over n launches, replayed from a graph
    (device time, not the host launch rate) unless --eager."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    g = None
    if not args.eager:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        g.replay()
        torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    if g is not None:
        g.replay()
    else:
        for _ in range(n):
            fn()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / n


def roofline(m) -> dict:
    """Roofline entry of the dominant unit: algorithmic bytes of the unit over
    its average duration against the HBM peak, the MFMA fraction beside it for
    the GEMM-shaped workloads, and the measured HBM traffic per launch (while
    it was taken on the current kernel sources)."""
    import traffic as traffic_store
    wl = m["wl"]
    achieved = m["avg_bytes"] / (m["avg_ms"] / 1e3) / 1e9
    tr = traffic_store.lookup(wl.name)
    out = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "frac_of_measured_ceiling": round(achieved / HBM_MEASURED_CEILING_GBS, 4),
        "traffic": tr["bytes_per_launch"] if tr else None,
        "kernel": m["kernel"],
        "avg_launch_us": round(m["avg_ms"] * 1e3, 2),
        "algo_bytes_per_launch": int(m["avg_bytes"]),
    }
    if m["cold_ms"] is not None:
        # the large-expert decode shares one layer's weights across its steps:
        # back-to-back steps can find hot experts in the 256 MB MALL, so the
        # HBM fraction is also given for steps after a 1 GiB write
        cold_achieved = m["avg_bytes"] / (m["cold_ms"] / 1e3) / 1e9
        out["frac_cold"] = round(cold_achieved / HBM_PEAK_GBS, 4)
    if wl.fmt != "w4a16" or wl.T >= 512:
        dt = "bf16" if wl.fmt == "w4a16" else "int8"
        out["mfma_frac"] = round(m["flops_per_call"] / (m["avg_ms"] / 1e3) / 1e12 / MFMA_PEAK[dt], 4)
    return out


def side_rows(m, torch, moe):
    """Router projection and expert-load telemetry on the workload's shape,
    timed alone: separate rows, not part of the step."""
    wl, bufs, units = m["wl"], m["bufs"], m["units"]
    tl = m["time_launches"]
    wr = torch.from_numpy(synth.router_weights(wl, 0).view(np.int16)).cuda()
    x0 = units[0][0]
    lg = torch.empty((wl.T, wl.E), dtype=torch.float32, device="cuda")
    router_us = tl(lambda: moe.router_logits(x0, wr, lg))
    router_bytes = wl.T * wl.H * 2 + wl.E * wl.H * 2 + wl.T * wl.E * 4
    router_row = {"kernel": "router_logits_kernel (moe_router_logits)",
                  "avg_launch_us": round(router_us, 2),
                  "algo_bytes_per_launch": router_bytes,
                  "achieved_GBps": round(router_bytes / (router_us * 1e-6) / 1e9, 1),
                  "flops_per_launch": 2 * wl.T * wl.H * wl.E}
    # one step's layers: their expert_offsets gathered into one [L, E + 1]
    # array, counts accumulated in one launch, each layer's 16 most-loaded
    # experts ranked
    step_units = m["schedule"][0]
    offs = torch.stack([bufs[u].offsets[:wl.E + 1] for u in step_units])
    loads = torch.zeros((len(step_units), wl.E), dtype=torch.int64, device="cuda")
    n_hot = min(16, wl.E)
    hot = torch.empty((len(step_units), n_hot), dtype=torch.int32, device="cuda")
    counts_us = tl(lambda: moe.expert_counts_accumulate(offs, loads))
    hot_us = tl(lambda: moe.expert_hot_rank(loads, n_hot, hot))
    telemetry_row = {"kernels": "expert_counts_kernel, hot_rank_kernel "
                                "(moe_expert_counts_accumulate, moe_expert_hot_rank)",
                     "layers": len(step_units), "hot_n": n_hot,
                     "counts_avg_launch_us": round(counts_us, 2),
                     "hot_rank_avg_launch_us": round(hot_us, 2)}
    return router_row, telemetry_row


def prefill_block(m) -> dict:
    """The prompt half of the metric: the grouped W8A8 FFN at T 4096."""
    wl = m["wl"]
    r = roofline(m)
    return {
        "workload": wl.name,
        "config": {"T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E, "k": wl.k, "format": "W8A8",
                   "layers_rotated": wl.units},
        "tokens_per_s": round(wl.T / (m["ms_per_step"] / 1e3), 1),
        "layer_us": round(m["ms_per_step"] * 1e3, 2),
        "ffn_us": r["avg_launch_us"],
        "mfma_frac": r["mfma_frac"],
        "mfma_peak_TOPs": MFMA_PEAK["int8"],
        "hbm_frac": r["frac"],
        "algo_bytes_per_launch": r["algo_bytes_per_launch"],
        "traffic": r["traffic"],
        "kernel": r["kernel"],
        "spread_median_layer_us": round(m["spread"]["median_ms_per_step"] * 1e3, 2),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(the layer path runs on a single GPU)", file=sys.stderr)
        sys.exit(2)
    import torch
    import quantized_moe_expert_top_amd as moe

    torch.cuda.set_device(0)
    moe.load()
    marker = Marker(args.mark)
    wl = synth.workload(args.workload)
    if args.units:
        wl = wl.with_(units=min(args.units, wl.units))
    m = measure(wl, args, torch, moe, marker, args.path)
    router_row, telemetry_row = side_rows(m, torch, moe)
    value = wl.T / (m["ms_per_step"] / 1e3)   # each step carries T tokens
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.fmt == "w4a16" else "int8",
        "data": "synthetic (seeded; random int4/int8 expert weights, N(0,1) activations)",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E, "k": wl.k,
                   "format": {"w4a16": "W4A16 g128",
                              "w4a8": "W4A8 (int4 g128 weights, int8 per-token activations)",
                              "w8a8": "W8A8"}[wl.fmt],
                   "layers_per_step": len(m["schedule"][0]),
                   "launch": "eager" if args.eager else "hip_graph_per_step",
                   "path": m["path"],
                   "mean_active_experts": round(m["mean_active"], 2),
                   "expert_rows": m["expert_rows"]},
        "roofline": roofline(m),
        "cpu_baseline": None,
        "spread": m["spread"],
        "router_projection": router_row,
        "expert_load_telemetry": telemetry_row,
        "wall_s_timed": round(m["wall"], 3),
    }
    if args.workload == "decode_t2" and not args.no_prefill and not args.units:
        del m
        torch.cuda.empty_cache()
        p = measure(synth.workload(PREFILL_WORKLOAD), args, torch, moe, marker)
        line["prefill"] = prefill_block(p)
        del p
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, layers_per_step(wl), args.cpu_budget_s)
    print(json.dumps(line), flush=True)


def cpu_baseline(wl, schedule, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of the same workload."""
    import oracle
    blas = "unknown BLAS"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in info) or blas
    except Exception:
        threads = 1
    cpu_model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 0
    done = 0
    el = 0.0
    arrs = None
    for u in range(wl.units):
        # inputs are generated before the clock starts; only the oracle is timed
        x, L = synth.x_bf16(wl, u), synth.router_logits(wl, u)
        if arrs is None or not wl.shared_weights:
            arrs = synth.layer_w8(wl, u) if wl.fmt == "w8a8" else synth.layer_w4(wl, u)
        get = lambda e, a=arrs: tuple(t[e] for t in a)  # noqa: E731
        t0 = time.perf_counter()
        if wl.fmt == "w4a16":
            oracle.moe_layer_w4a16(x, L, wl.k, get)
        elif wl.fmt == "w4a8":
            oracle.moe_layer_w4a8(x, L, wl.k, get)
        else:
            oracle.moe_layer_w8a8(x, L, wl.k, get)
        el += time.perf_counter() - t0
        done += 1
        if el > budget_s:
            break
    per_unit = el / done
    per_step = per_unit * len(schedule[0])
    return {
        "value": round(wl.T / per_step, 4),
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{done} of {wl.units} units of workload {wl.name} through the float64 numpy "
                   f"oracle (input generation excluded); "
                   f"{per_unit:.3f} s per unit, scaled to {len(schedule[0])} units per step; "
                   f"{cpu_model}, {affinity} cores in the affinity mask, {blas}"),
    }


if __name__ == "__main__":
    main()
