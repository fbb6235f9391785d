"""Benchmark of the MoE dispatch/combine hot path on one MI355X.

One step = one pass of the whole path over one layer's batch:
  moe_route_build (multihot map, counts, padded offsets, rows of slots; the
  eager readback included) + moe_dispatch + moe_combine + moe_combine_bwd
  (cached dispatch of grad_out plus the routing-weight gradients).

Protocol (after the benchmark section of "Add the deepep expert-parallel
implementation": distinct layers back to back):
  * `--sets` (default 4) independent layer buffer sets, each with its own
    routing, rotated step by step so a step's inputs were last touched several
    hundred MB of traffic earlier (MI355X's 256 MB Infinity Cache);
  * combine reads its own expert-output buffer Y (a stand-in for the grouped
    GEMM output) and the backward reads another one, F (the expert output
    before the routing weight), so no kernel of a step re-reads what an
    earlier kernel of the same step left in cache;
  * W warm-up steps; K untimed steps with every call's kernels timed (the
    per-kernel breakdown, which picks the dominant kernel); then the timed
    region: K steps between two device synchronizations, with only the
    dominant call timed.  Timing is the library's moe_time_next_call with
    fence-free events (binding.KernelTimer): the events ride on the call's own
    kernel launches, so no event packet enters the stream.
  * eager steps route and dispatch in one call (moe_route_dispatch) into the
    set's worst-case-sized buffers: the dispatch is queued before the row
    count is read back, so the device does not wait for the host between the
    two.  The per-kernel breakdown times the route and the dispatch as two
    calls (the same kernels on the same inputs); sync-free steps always use two
    calls, with the dispatch through binding.PreparedDispatch.  The combine
    and its backward go through binding.PreparedCombine / PreparedCombineBwd
    (buffers checked once, each step passes its row count), which keeps the
    host's work between the eager readback and their launches small.

Output: one JSON line.  `value` = algorithmic bytes of the step / wall time of
the step (GB/s); `roofline` gives the dominant kernel's algorithmic GB/s
(from its device time, average and spread over the timed steps) against
MI355X's 8 TB/s, and against ceilings measured in the same run:
  * `ceiling_GBps` / `frac_of_ceiling`: a one-shot copy of 1 GiB in address
    order with non-temporal stores (libmoe_ceiling), the best plain stream
    that moves as many bytes in as out;
  * `write_bound_us` / `frac_of_write_bound`: the time the reference kernels
    take to write the kernel's output rows alone, in the same layout and
    store order and reading nothing (a token-major scatter of the data rows,
    plus a one-shot fill of the sync-free zero tail);
  * `hip_copy_GBps`: the HIP runtime's own 1 GiB device copy (torch copy_).
The combine also carries `gather_read_us` / `gather_us`: a plain reference
gather of the same rows along the same handle, reading only, then also writing
the summed rows; `frac_of_gather(_read)` = that time / the combine's.
`cpu_baseline` times the oracle on the host on a bounded sample of the same
workload.  `next` times, outside the step, the FP8 dispatch and the dispatch
backward on the same routings.  The metric is quoted at 4096 and at 16384
tokens; `also` repeats the step (value, roofline, per-kernel times) on every
other workload of the benchmark description after the main one
(`--companions`): the tiny layer, the 16384-token H = 4096 layers and the
skewed layer.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch+combine µs/layer and achieved HBM GB/s (% peak), 4096 & 16384 tok"
PEAK_GBS = 8000.0  # MI355X HBM3E


def byte_model(wl, tpe_total_valid, R, n_active, idx_bytes, with_probs):
    """Algorithmic bytes per launch (each input read once, each output written once)."""
    T, H, k, E = wl.T, wl.H, wl.k, wl.E
    EL = wl.num_local
    row = 2 * H
    route = (T * k * idx_bytes + T * E            # ids in, multihot map out
             + (T * k * 4 + T * E * 4 if with_probs else 0)  # weights in, probs out
             + T * k * 4                           # row_of_slot out
             + (2 * EL + 1) * 4 + 16)              # counts, offsets, status
    dispatch = (n_active * row + T * k * 4 * 2     # active token rows, weights, row_of_slot
                + R * row + R * 12)                # rows out + row_w/row_token/row_expert
    combine = tpe_total_valid * row + T * k * 4 + T * row
    bwd = (n_active * row + tpe_total_valid * row  # grad_out rows in, expert rows in
           + T * k * 4 + R * row + T * k * 4)      # row_of_slot, grad rows out, dw out
    return {"route": route, "dispatch": dispatch, "combine": combine, "combine_bwd": bwd}


def byte_model_next(wl, data_rows, R, n_active):
    """Algorithmic bytes per launch of the two calls outside the step: the FP8
    dispatch (codes plus one fp32 scale per 128 elements) and the dispatch
    backward (the combine of the grad rows plus the weight-gradient gather)."""
    T, H, k = wl.T, wl.H, wl.k
    fp8 = (n_active * 2 * H + T * k * 4 * 2
           + R * H + R * (H // 128) * 4 + R * 12)
    dbwd = (data_rows * 2 * H + T * k * 4 * 2     # grad rows in, row_of_slot, grad_row_w
            + T * 2 * H + T * k * 4)               # grad_x out, grad_topk_w out
    return {"dispatch_fp8": fp8, "dispatch_bwd": dbwd}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_30b_a3b")
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall budget of the oracle CPU-baseline leg (0 = skip)")
    ap.add_argument("--companions", default="tiny,h4096_rank_share,skewed,backward_h4096",
                    help="workloads also timed (value and roofline only) after the main one; "
                         "'' for none")
    ap.add_argument("--no-next", action="store_true",
                    help="skip timing the FP8 dispatch and the dispatch backward")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-sized layers replayed from a HIP graph")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 8 plain device-to-device copies of MIB MiB (torch copy_) and "
                         "exit: the reference kernel for scaling HBM traffic counters")
    ap.add_argument("--cpu-worker", nargs=3, metavar=("DIR", "SECONDS", "WORKLOAD"),
                    help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_worker:
        cpu_worker(args.cpu_worker[0], float(args.cpu_worker[1]), args.cpu_worker[2])
        return
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU's share only (no inter-GPU exchange is built); "
              f"--gpus {args.gpus} is not supported, run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from combine_topk_idx_multihot_amd import binding as B
    from combine_topk_idx_multihot_amd import inputs

    B.moe_device_check(0)
    # ceilings beside the 8 TB/s peak, measured on this machine before the layers
    ceil = stream_ceilings(torch, torch.cuda.current_stream())
    result, sets, wl = measure(args.workload, args, not args.no_next, torch, B, inputs, ceil)
    result["ceilings"] = ceil
    # the row kernels' workgroup numbering assumes workgroup j runs on XCD j mod 8
    from combine_topk_idx_multihot_amd import ceiling as C
    result["xcd_round_robin"] = C.xcd_round_robin()

    # ---- CPU baseline: the oracle on the host, bounded sample ---------------
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(wl, sets[0], args.cpu_seconds, torch)
    del sets

    # ---- the metric's 16384-token layers, alongside the 4096-token one -------
    comp = [c for c in args.companions.split(",") if c and c != args.workload]
    if comp:
        result["also"] = {}
        for name in comp:
            torch.cuda.empty_cache()
            r, s_, _ = measure(name, args, False, torch, B, inputs, ceil)
            del s_
            result["also"][name] = {k: r[k] for k in ("value", "unit", "ms_per_step", "config",
                                                      "us_per_layer", "kernels", "roofline")}

    # ---- decode-sized layers replayed from a captured HIP graph --------------
    if not args.no_decode:
        torch.cuda.empty_cache()
        result["decode_graph"] = decode_graph(torch, B, inputs)
    print(json.dumps(result), flush=True)


def measure(name, args, with_next, torch, B, inputs, ceil):
    """Warm up, take the per-kernel breakdown, then time K steps of workload
    `name`; `ceil` holds the stream ceilings of this machine.  Returns (result
    fields, buffer sets, workload)."""
    wl = inputs.WORKLOADS[name]
    seed0 = args.seed if args.seed is not None else 1000 + list(inputs.WORKLOADS).index(wl.name) + 1
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    EL = wl.num_local
    mode = B.MOE_SYNC_FREE if wl.sync_free else B.MOE_EAGER
    d = B.make_desc(wl.T, wl.k, wl.E, wl.lb, EL, wl.P, mode, False, wl.cap if wl.sync_free else 0)
    Rmax = B.moe_capacity_min(d) if not wl.sync_free else wl.cap
    H = wl.H

    # ---- buffer sets -------------------------------------------------------
    sets = []
    gen = torch.Generator(device=dev)
    for s in range(args.sets):
        idx, w = inputs.make_routing(wl, seed0 + 7919 * s)
        gen.manual_seed(seed0 * 31 + s)
        st = {
            "idx_np": idx, "w_np": w,
            "idx": torch.from_numpy(idx).to(dev), "w": torch.from_numpy(w).to(dev),
            "x": torch.randn((wl.T, H), generator=gen, device=dev).to(torch.bfloat16),
            "g": torch.randn((wl.T, H), generator=gen, device=dev).to(torch.bfloat16),
            "Y": torch.randn((Rmax, H), generator=gen, device=dev).to(torch.bfloat16),
            "F": torch.randn((Rmax, H), generator=gen, device=dev).to(torch.bfloat16),
            "rows": torch.empty((Rmax, H), dtype=torch.bfloat16, device=dev),
            "grad_rows": torch.empty((Rmax, H), dtype=torch.bfloat16, device=dev),
            "row_w": torch.empty(Rmax, dtype=torch.float32, device=dev),
            "row_token": torch.empty(Rmax, dtype=torch.int32, device=dev),
            "row_expert": torch.empty(Rmax, dtype=torch.int32, device=dev),
            "out": torch.empty((wl.T, H), dtype=torch.bfloat16, device=dev),
            "dw": torch.empty((wl.T, wl.k), dtype=torch.float32, device=dev),
            "probs": torch.empty((wl.T, wl.E), dtype=torch.float32, device=dev),
            "h": B.alloc_handle(d, dev),
        }
        # the dispatch right after the eager readback is on the step's critical
        # path: its buffers are checked once, and each step passes only R
        st["dispatch"] = B.PreparedDispatch(d, st["h"], st["x"], H, st["rows"], st["w"],
                                            st["row_w"], st["row_token"], st["row_expert"],
                                            stream=stream)
        # the combine and its backward, checked once likewise: after the eager
        # readback the host has only the dispatch's run time to issue them
        st["combine"] = B.PreparedCombine(d, st["h"], st["Y"], H, st["out"], stream=stream)
        st["combine_bwd"] = B.PreparedCombineBwd(d, st["h"], st["g"], H, st["grad_rows"], st["F"],
                                                 st["dw"], stream=stream)
        sets.append(st)
    torch.cuda.synchronize()

    names = ("route", "dispatch", "combine", "combine_bwd")

    def step(st, timed=None):
        """One pass of the path; timed = {call name: KernelTimer} times those
        calls' kernels on their own dispatch packets (no event packet enters
        the stream)."""
        t = timed or {}
        if wl.sync_free or "route" in t or "dispatch" in t:
            # two calls: sync-free never waits, and the breakdown times each
            if "route" in t:
                t["route"].arm()
            B.moe_route_build(d, st["idx"], st["h"], st["w"], st["probs"], stream=stream)
            R = wl.cap if wl.sync_free else st["h"].total
            if "dispatch" in t:
                t["dispatch"].arm()
            st["dispatch"](R)
        else:
            # eager: one call, whose dispatch is queued before the readback
            B.moe_route_dispatch(d, st["idx"], st["h"], st["x"], H, st["rows"], st["w"],
                                 st["probs"], st["row_w"], st["row_token"], st["row_expert"],
                                 stream=stream)
            R = st["h"].total
        if "combine" in t:
            t["combine"].arm()
        st["combine"](R)
        if "combine_bwd" in t:
            t["combine_bwd"].arm()
        st["combine_bwd"](R)
        return R

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()

    # per-set routing facts for the byte model (from the warmed handles)
    facts = []
    for st in sets:
        step(st)
        torch.cuda.synchronize()
        hs = st["h"].status.cpu().numpy()
        idx = st["idx_np"]
        local = (idx >= wl.lb) & (idx < wl.lb + EL)
        n_active = int(local.any(axis=1).sum())
        R = wl.cap if wl.sync_free else int(hs[0])
        facts.append(byte_model(wl, int(hs[2]), R, n_active, 4, True)
                     | byte_model_next(wl, int(hs[2]), R, n_active) | {"R": R})

    # breakdown pass (untimed): every call's kernels timed; picks the
    # dominant kernel
    evs = [{n: B.KernelTimer(stream) for n in names} for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(sets[i % len(sets)], evs[i])
    torch.cuda.synchronize()
    kern = {}
    for n in names:
        ms = [evs[i][n].elapsed_ms() for i in range(args.steps)]
        b = float(np.mean([facts[i % len(sets)][n] for i in range(args.steps)]))
        avg = float(np.mean(ms))
        kern[n] = {"avg_us": round(avg * 1e3, 2), "median_us": round(float(np.median(ms)) * 1e3, 2),
                   "alg_bytes": int(b), "GBps": round(b / (avg * 1e-3) / 1e9, 1)}
    dominant = max(("dispatch", "combine", "combine_bwd"), key=lambda n: kern[n]["avg_us"])

    # timed region: K steps between two synchronizations; the dominant
    # call's kernels timed live on their launch stream
    dev_ = [B.KernelTimer(stream) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % len(sets)], {dominant: dev_[i]})
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    step_bytes = float(np.mean([sum(facts[i % len(sets)][n] for n in names)
                                for i in range(args.steps)]))
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dom_all = np.array([t.elapsed_ms() for t in dev_]) * 1e3
    # whole steps back to back on the device: dominant-call start to the next
    # step's, in (up to) 5 contiguous windows, and the median of the windows
    per_step = np.array([dev_[i + 1].since_ms(dev_[i]) for i in range(args.steps - 1)]) * 1e3
    windows = ([float(np.mean(w)) for w in np.array_split(per_step, min(5, len(per_step)))]
               if len(per_step) else [])
    dom_ms = float(np.mean(dom_all)) * 1e-3
    dom_bytes = float(np.mean([facts[i % len(sets)][dominant] for i in range(args.steps)]))
    dom_gbs = dom_bytes / (dom_ms * 1e-3) / 1e9
    dev_us = sum(kern[n]["avg_us"] for n in names)

    # the write bound of every row kernel: the reference kernels writing the
    # same output rows alone (same layout and store order, nothing read)
    wb = write_bounds(wl, sets, facts, args.steps, torch, wl.k * wl.num_local >= 2 * wl.E)
    for n in ("dispatch", "combine", "combine_bwd"):
        kern[n]["frac_of_ceiling"] = round(kern[n]["GBps"] / ceil["copy_GBps"], 4)
    for n in ("dispatch", "combine_bwd"):  # both write the layer's rows token-major
        kern[n]["write_bound_us"] = wb
        kern[n]["frac_of_write_bound"] = round(wb / kern[n]["avg_us"], 4)
    # the combine against the reference gather of its rows: read only, and
    # with the summed rows written
    g_read, g_write = gather_bounds(sets, facts, args.steps, torch)
    kern["combine"]["gather_read_us"] = g_read
    kern["combine"]["gather_us"] = g_write
    kern["combine"]["frac_of_gather"] = round(g_write / kern["combine"]["avg_us"], 4)
    kern["combine"]["frac_of_gather_read"] = round(g_read / kern["combine"]["avg_us"], 4)

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "H": H, "E": wl.E, "k": wl.k,
                   "local_experts": EL, "pad_multiple": wl.P,
                   "mode": "sync_free" if wl.sync_free else "eager",
                   "rows": int(np.mean([f["R"] for f in facts])), "buffer_sets": args.sets},
        "us_per_layer": {"forward_device": round(kern["route"]["avg_us"] + kern["dispatch"]["avg_us"] + kern["combine"]["avg_us"], 2),
                         "backward_device": kern["combine_bwd"]["avg_us"],
                         "step_wall": round(ms_per_step * 1e3, 2), "step_device": round(dev_us, 2),
                         # the metric's pair: dispatch + combine, their algorithmic bytes
                         # over their summed device time
                         "dispatch_combine": dispatch_combine(kern),
                         "step_windows": {"us_per_step": [round(w, 2) for w in windows],
                                          "median_us_per_step": round(float(np.median(windows)), 2)
                                          if windows else None}},
        "kernels": kern,
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(dom_gbs, 1),
                     "peak": PEAK_GBS, "unit": "GB/s", "frac": round(dom_gbs / PEAK_GBS, 4),
                     "traffic": None, "avg_us": round(dom_ms * 1e3, 2),
                     "spread_us": {"median": round(float(np.median(dom_all)), 2),
                                   "min": round(float(dom_all.min()), 2),
                                   "p10": round(float(np.percentile(dom_all, 10)), 2),
                                   "p90": round(float(np.percentile(dom_all, 90)), 2),
                                   "max": round(float(dom_all.max()), 2)},
                     "frac_median": round(dom_bytes / (float(np.median(dom_all)) * 1e-6) / 1e9
                                          / PEAK_GBS, 4),
                     "alg_bytes_per_launch": int(dom_bytes),
                     "ceiling_GBps": ceil["copy_GBps"],
                     "frac_of_ceiling": round(dom_gbs / ceil["copy_GBps"], 4),
                     "hip_copy_GBps": ceil["hip_copy_GBps"],
                     "frac_of_hip_copy": round(dom_gbs / ceil["hip_copy_GBps"], 4)},
    }
    if dominant in ("dispatch", "combine_bwd"):
        result["roofline"]["write_bound_us"] = wb
        result["roofline"]["frac_of_write_bound"] = round(wb / (dom_ms * 1e3), 4)

    result["roofline"]["traffic"] = measured_traffic(wl.name, dominant)
    if with_next:
        result["next"] = time_next(wl, d, sets, facts, args.steps, stream, torch, B, kern)
    return result, sets, wl


def time_next(wl, d, sets, facts, steps, stream, torch, B, kern):
    """The FP8 dispatch and the dispatch backward over the same buffer sets
    (handles as routed by the step), each call's kernels timed by the library
    (moe_time_next_call)."""
    H, T, k = wl.H, wl.T, wl.k
    dev = sets[0]["x"].device
    gen = torch.Generator(device=dev)
    for s_i, st in enumerate(sets):
        R = st["rows"].shape[0]
        gen.manual_seed(4242 + s_i)
        st["rows_q"] = torch.empty((R, H), dtype=torch.uint8, device=dev)
        st["row_scale"] = torch.empty((R, H // 128), dtype=torch.float32, device=dev)
        st["grad_row_w"] = torch.randn(R, generator=gen, device=dev)
        st["grad_x"] = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        st["grad_topk_w"] = torch.empty((T, k), dtype=torch.float32, device=dev)

    def run(i, ev=None):
        st, f = sets[i % len(sets)], facts[i % len(sets)]
        R = f["R"]
        if ev is not None:
            ev[0].arm()
        B.moe_dispatch_fp8(d, st["h"], st["x"], H, R, st["rows_q"], st["row_scale"], st["w"],
                           st["row_w"], st["row_token"], st["row_expert"], stream=stream)
        if ev is not None:
            ev[1].arm()
        # grad rows: the F buffer (independent of every other input here)
        B.moe_dispatch_bwd(d, st["h"], st["F"], H, R, st["grad_x"], st["grad_row_w"],
                           st["grad_topk_w"], stream=stream)

    for i in range(2):
        run(i)
    evs = [(B.KernelTimer(stream), B.KernelTimer(stream)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        run(i, evs[i])
    torch.cuda.synchronize()
    out = {}
    for j, n in enumerate(("dispatch_fp8", "dispatch_bwd")):
        ms = [evs[i][j].elapsed_ms() for i in range(steps)]
        b = float(np.mean([facts[i % len(sets)][n] for i in range(steps)]))
        avg = float(np.mean(ms))
        out[n] = {"avg_us": round(avg * 1e3, 2), "median_us": round(float(np.median(ms)) * 1e3, 2),
                  "alg_bytes": int(b), "GBps": round(b / (avg * 1e-3) / 1e9, 1),
                  "frac_of_peak": round(b / (avg * 1e-3) / 1e9 / PEAK_GBS, 4)}
    out["dispatch_fp8"]["time_vs_bf16_dispatch"] = round(
        out["dispatch_fp8"]["avg_us"] / kern["dispatch"]["avg_us"], 3)
    return out


def kernel_source_sha256():
    import glob
    import hashlib

    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "combine_topk_idx_multihot_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (profiles/traffic.json, counters scaled by a plain copy
    of known size); None if there is none for this workload or if the kernel
    sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_sha256():
        return None
    k = t.get("workloads", {}).get(workload, {}).get(kernel)
    return None if k is None else int(k["bytes"])


def calibrate_copy(mib):
    """Plain copies of a known size: each launch reads and writes `mib` MiB, so
    a traffic counter's reading for it gives the counter's scale."""
    import torch

    n = mib * (1 << 20)
    bufs = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(4)]
    for b in bufs:
        b.fill_(1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(8):
        bufs[(2 * i + 1) % 4].copy_(bufs[(2 * i) % 4])
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 8
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                      "launches": 8, "GBps": round(2 * n / dt / 1e9, 1)}), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


DECODE_SHAPES = ((1, 2048), (256, 2048), (1, 4096), (256, 4096))


def _graph_us(torch, fn, reps):
    """fn(stream) captured once in a HIP graph, then replayed `reps` times
    back to back: us per replay, from events around the replays."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(s)  # eager warm-up on the capture stream
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        g.capture_begin()
        fn(s)
        g.capture_end()
        for _ in range(10):
            g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(s)
        for _ in range(reps):
            g.replay()
        e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del g
    return us


def decode_graph(torch, B, inputs, reps=100, layers=(1, 4, 16)):
    """Decode-sized layers: route + dispatch (moe_route_dispatch) + combine in
    sync-free mode (worst-case rows, nothing read back to the host), E = 128,
    top-8, on a
    one-rank share of 32 experts (expert parallelism over 4 GPUs).  As on the
    pages' benchmark, distinct layers (each with its own routing, tokens and
    buffers) run back to back: L of them are captured in one HIP graph and the
    graph is replayed; us per layer = us per replay / L.  The pages time four
    layers, so `us_per_layer` is L = 4; L = 1 and 16 are listed beside it.  A
    graph replay has a fixed cost of its own on the host and GPU side, which
    `graph_floor_us` shows: one replay of a graph of one trivial kernel.  The
    captured work is the library's kernels only (no exchange, no experts)."""
    E, k, EL, P = 128, 8, 32, 1
    out = {"shape": {"E": E, "k": k, "local_experts": EL, "pad_multiple": P,
                     "mode": "sync_free", "replays": reps, "layers_per_graph": list(layers)}}
    z = torch.zeros(256, device="cuda")
    out["graph_floor_us"] = round(_graph_us(torch, lambda s: z.add_(1.0), reps), 2)
    for T, H in DECODE_SHAPES:
        lay = []
        for li in range(max(layers)):
            rng = np.random.default_rng([77, T, H, li])
            idx, w = inputs.topk_softmax(T, E, k, rng)
            C = B.moe_capacity_min(B.make_desc(T, k, E, 0, EL, P, B.MOE_EAGER, False, 0))
            d = B.make_desc(T, k, E, 0, EL, P, B.MOE_SYNC_FREE, False, C)
            gen = torch.Generator(device="cuda")
            gen.manual_seed(77 * T + H + 1000 * li)
            lay.append(dict(
                d=d, C=C, idx=torch.from_numpy(idx).cuda(), w=torch.from_numpy(w).cuda(),
                x=torch.randn((T, H), generator=gen, device="cuda").to(torch.bfloat16),
                h=B.alloc_handle(d), rows=torch.empty((C, H), dtype=torch.bfloat16, device="cuda"),
                row_w=torch.empty(C, dtype=torch.float32, device="cuda"),
                y=torch.empty((T, H), dtype=torch.bfloat16, device="cuda")))

        def run(s, n, H=H, lay=lay):
            for o in lay[:n]:
                # route + dispatch in one call (one launch when T*k <= 16)
                B.moe_route_dispatch(o["d"], o["idx"], o["h"], o["x"], H, o["rows"], o["w"],
                                     None, o["row_w"], stream=s)
                B.moe_combine(o["d"], o["h"], o["rows"], H, o["C"], o["y"], stream=s)

        per = {L: round(_graph_us(torch, lambda s, L=L: run(s, L), reps) / L, 2) for L in layers}
        out[f"T{T}_H{H}"] = {"us_per_layer": per[4] if 4 in per else per[layers[0]],
                             **{f"L{L}_us_per_layer": v for L, v in per.items()}}
        del lay
    return out


def dispatch_combine(kern):
    """Dispatch + combine of one layer: summed device time (breakdown pass),
    their algorithmic bytes over it, and the fraction of the HBM peak."""
    us = kern["dispatch"]["avg_us"] + kern["combine"]["avg_us"]
    nbytes = kern["dispatch"]["alg_bytes"] + kern["combine"]["alg_bytes"]
    gbs = nbytes / (us * 1e-6) / 1e9 if us > 0 else 0.0
    return {"us": round(us, 2), "GBps": round(gbs, 1), "frac": round(gbs / PEAK_GBS, 4)}


def _events_ms(torch, stream, fn, reps):
    """Average ms of fn() over reps back-to-back calls, by events on `stream`."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(reps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def stream_ceilings(torch, stream, mib=1024, reps=6):
    """Plain streams over `mib` MiB buffers, timed live, in GB/s of bytes read +
    written: the one-shot copy and zero fill of libmoe_ceiling (1 KiB per
    wave, address order, non-temporal stores) and the HIP runtime's device
    copy (torch copy_)."""
    from combine_topk_idx_multihot_amd import ceiling as C

    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    C.copy(a, b)
    C.fill(b)
    ms_copy = _events_ms(torch, stream, lambda i: C.copy(a if i % 2 == 0 else b,
                                                          b if i % 2 == 0 else a), reps)
    ms_fill = _events_ms(torch, stream, lambda i: C.fill(a if i % 2 == 0 else b), reps)
    ms_hip = _events_ms(torch, stream, lambda i: (b if i % 2 == 0 else a).copy_(
        a if i % 2 == 0 else b), reps)
    del a, b
    return {"copy_GBps": round(2 * n / (ms_copy * 1e-3) / 1e9, 1),
            "fill_GBps": round(n / (ms_fill * 1e-3) / 1e9, 1),
            "hip_copy_GBps": round(2 * n / (ms_hip * 1e-3) / 1e9, 1),
            "bytes": n, "kind": "libmoe_ceiling one-shot copy and fill, 1 KiB per wave; "
                                "torch copy_"}


def write_bounds(wl, sets, facts, steps, torch, dense):
    """us per layer for the reference kernels to write the layer's output rows
    alone: a token-major scatter of zeros to the rows each set's handle names
    (the dispatch's store order and segment size), plus, in sync-free mode, a
    one-shot fill of the zero tail past the set's routed total.  Pad rows
    (at most P - 1 per expert) are left out.  Rotates over the sets like the
    step; average over `steps` calls."""
    from combine_topk_idx_multihot_amd import ceiling as C

    seg = 1 if dense else 2  # the dispatch's copy segment (1 KiB on dense layers)
    stream = torch.cuda.current_stream()
    totals = [int(st["h"].status[0]) for st in sets]

    def one(i):
        st = sets[i % len(sets)]
        R = facts[i % len(sets)]["R"]
        C.scatter(st["h"].row_of_slot, st["rows"][:R], seg_kib=seg)
        tot = totals[i % len(sets)]
        if wl.sync_free and tot < R:
            C.fill(st["rows"][tot:R])

    one(0)
    return round(_events_ms(torch, stream, one, steps) * 1e3, 2)


def gather_bounds(sets, facts, steps, torch):
    """us per layer for the reference gather of the combine's rows along each
    set's handle (the combine's segment size and load batches): read only,
    then with the summed rows written to the set's output.  Rotates over the
    sets like the step; average over `steps` calls."""
    from combine_topk_idx_multihot_amd import ceiling as C

    H = sets[0]["Y"].shape[1]
    seg = 1 if H < 1024 else 2  # the combine's segment (KiB)
    stream = torch.cuda.current_stream()
    sink = torch.zeros(1, dtype=torch.int32, device=sets[0]["Y"].device)

    def run(i, write):
        st = sets[i % len(sets)]
        R = facts[i % len(sets)]["R"]
        C.gather(st["h"].row_of_slot, st["Y"][:R], st["out"] if write else None,
                 None if write else sink, seg_kib=seg)

    run(0, False)
    r = _events_ms(torch, stream, lambda i: run(i, False), steps)
    run(0, True)
    w = _events_ms(torch, stream, lambda i: run(i, True), steps)
    return round(r * 1e3, 2), round(w * 1e3, 2)


def oracle_steps(wl, a, budget_s, max_reps=500):
    """Full steps of the single-threaded C oracle (route with the dispatched
    rows, combine, combine backward with dw) on one layer's arrays, for about
    budget_s seconds.  Returns (steps, seconds, algorithmic bytes)."""
    import oracle

    idx, w, x, g, Y, F = (a[n] for n in ("idx", "w", "x", "g", "Y", "F"))
    EL = wl.num_local
    C = wl.cap if wl.sync_free else 0
    local = (idx >= wl.lb) & (idx < wl.lb + EL)
    n_active = int(local.any(axis=1).sum())
    reps, t_used, bytes_done = 0, 0.0, 0
    while t_used < budget_s and reps < max_reps:
        t0 = time.perf_counter()
        r = oracle.route(idx, wl.E, wl.lb, EL, wl.P, sync_free=wl.sync_free, C=C, w=w, x=x,
                         want_probs=True)
        oracle.combine(idx, r.row_of_slot, Y[:r.R], wl.E, wl.lb, EL)
        oracle.combine_bwd(idx, r.row_of_slot, r.row_token, g, wl.E, wl.lb, EL, F=F[:r.R], R=r.R)
        t_used += time.perf_counter() - t0
        bm = byte_model(wl, int(r.tpe.sum()), r.R, n_active, 4, True)
        bytes_done += sum(bm.values())
        reps += 1
    return reps, t_used, bytes_done


def cpu_worker(arg_dir, budget_s, wname):
    """One process of the all-cores leg: the arrays come memory-mapped from
    arg_dir (no torch, no GPU); prints one JSON line."""
    from combine_topk_idx_multihot_amd import inputs

    a = {n: np.load(os.path.join(arg_dir, n + ".npy"), mmap_mode="r")
         for n in ("idx", "w", "x", "g", "Y", "F")}
    reps, t_used, bytes_done = oracle_steps(inputs.WORKLOADS[wname], a, budget_s)
    print(json.dumps({"steps": reps, "seconds": t_used, "bytes": bytes_done}), flush=True)


def host_cores():
    """Cores this process may run on, at most 16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(wl, st, budget_s, torch):
    """The oracle on the host, on a bounded sample of the same layer: one
    thread in this process, then one unchanged single-threaded oracle per
    host core in child processes (aggregate rate over their common wall
    time)."""
    import subprocess
    import tempfile

    u16 = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    a = {"idx": np.ascontiguousarray(st["idx_np"]), "w": np.ascontiguousarray(st["w_np"]),
         "x": u16(st["x"]), "g": u16(st["g"]), "Y": u16(st["Y"]), "F": u16(st["F"])}
    reps, t_used, bytes_done = oracle_steps(wl, a, budget_s)
    out = {"value": round(bytes_done / t_used / 1e9, 3), "unit": "GB/s", "cores": 1,
           "kind": "oracle",
           "ms_per_step": round(t_used * 1e3 / reps, 1),
           "host": {"cpu_model": cpu_model(), "logical_cpus": os.cpu_count()},
           "sample": f"{reps} full step(s) of the {wl.name} layer (route+dispatch+combine+"
                     f"combine_bwd with dw), single-threaded C oracle, {t_used:.1f} s"}

    n = host_cores()
    budget_all = max(2.0, budget_s / 2)
    shm = "/dev/shm" if os.path.isdir("/dev/shm") else None
    with tempfile.TemporaryDirectory(prefix="moe_oracle_", dir=shm) as d:
        for k, v in a.items():
            np.save(os.path.join(d, k + ".npy"), v)
        del a
        wall0 = time.perf_counter()
        procs = [subprocess.Popen([sys.executable, os.path.abspath(__file__), "--cpu-worker", d,
                                   str(budget_all), wl.name],
                                  stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
                 for _ in range(n)]
        res = []
        for p in procs:
            so, se = p.communicate(timeout=budget_all * 10 + 120)
            if p.returncode != 0:
                raise RuntimeError(f"oracle worker failed ({p.returncode}): {se[-500:]}")
            res.append(json.loads(so.strip().splitlines()[-1]))
        wall = time.perf_counter() - wall0
    span = max(r["seconds"] for r in res)
    steps = sum(r["steps"] for r in res)
    out["all_cores"] = {
        "value": round(sum(r["bytes"] for r in res) / span / 1e9, 3), "unit": "GB/s",
        "cores": n, "processes": n,
        "ms_per_step": round(span * 1e3 * n / steps, 1),
        "sample": f"{n} processes, each the single-threaded C oracle on its own full steps of "
                  f"the same layer (memory-mapped inputs): {steps} steps in {span:.1f} s of "
                  f"oracle time ({wall:.1f} s wall with start-up); rate = all their bytes / the "
                  f"longest process's oracle time"}
    return out


if __name__ == "__main__":
    main()
