"""bench.py's host logic on the CPU: the one-GPU guard, and the algorithmic
byte model held against the HBM traffic the hardware counters measured.

profiles/traffic.json holds rocprofv3 FETCH_SIZE / WRITE_SIZE per launch of
every call on the five measured layers, scaled by a plain copy of known size.
The byte model counts each input once and each output once.  The row kernels
over-write nothing and, walking tokens, re-read nothing, so the two must agree
closely; a mistake in the model (a dropped metadata array, rows counted for
the wrong R, the FP8 scales forgotten) shows up as a mismatch of several
percent.  The one known excess: a dispatch or combine backward that walks the
route's row list keeps a tile of about 512 token rows in each XCD's L2 while
it writes; at H = 4096 that tile (4 MB) is as large as the L2, and some token
rows are fetched again (counted 1.13 and 1.10 times the model at 16384
tokens; 2048-wide rows, a 2 MB tile, stay within 1 %).  The routing facts
(data rows, padded rows, active tokens) come from the same seeded generators
the benchmark uses.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from combine_topk_idx_multihot_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROW_CALLS = ("dispatch", "combine", "combine_bwd", "dispatch_bwd", "dispatch_fp8")


def traffic():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        return json.load(fh)


def routing_facts(wl, seed):
    """(data rows, rows R, tokens with a local slot) of one seeded routing."""
    idx, _ = inputs.make_routing(wl, seed)
    lb, EL = wl.lb, wl.num_local
    tpe = np.array([(idx == lb + e).any(axis=1).sum() for e in range(EL)], np.int64)
    data = int(tpe.sum())
    R = wl.cap if wl.sync_free else int(((tpe + wl.P - 1) // wl.P * wl.P).sum())
    n_active = int(((idx >= lb) & (idx < lb + EL)).any(axis=1).sum())
    return data, R, n_active


def model_bytes(wname, sets=4):
    """The benchmark's byte model averaged over its buffer sets (same seeds)."""
    wl = inputs.WORKLOADS[wname]
    seed0 = 1000 + list(inputs.WORKLOADS).index(wname) + 1
    acc = {}
    for s in range(sets):
        data, R, n_active = routing_facts(wl, seed0 + 7919 * s)
        m = bench.byte_model(wl, data, R, n_active, 4, True) | bench.byte_model_next(wl, data, R,
                                                                                   n_active)
        for k, v in m.items():
            acc[k] = acc.get(k, 0.0) + v / sets
    return acc


def route_blocks(T, k, EL):
    """The library's count of route blocks: blocks of 512 slots up to 512
    local experts (else 256), or one block of up to 2048 slots when its
    local experts are few (T <= 1024 // k with EL <= 256, or T <= 2048 // k
    with EL <= 64)."""
    if T == 0:
        return 0
    nblk = -(-T // ((512 if EL <= 512 else 256) // k))
    if nblk > 1 and (T <= 1024 // k and EL <= 256 or T <= 2048 // k and EL <= 64):
        return 1
    return nblk


def walks_list(wl):
    """The library's rule for writing the row list (see moe_route_workspace_size)."""
    EL = wl.num_local
    nblk = route_blocks(wl.T, wl.k, EL)
    return nblk > 1 and nblk * EL <= 65536 and wl.k * EL >= 2 * wl.E


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


@pytest.mark.parametrize("wname", sorted(traffic()["workloads"]))
def test_byte_model_matches_counted_traffic(wname):
    meas = traffic()["workloads"][wname]
    model = model_bytes(wname)
    # Each launch also fetches its code and arguments (tens of KB that the
    # counters see and the model does not): only a layer of well under a MB
    # per call, the tiny one, notices, hence the absolute slack.
    slack = 256 << 10
    wl = inputs.WORKLOADS[wname]
    lists = walks_list(wl)
    token_bytes = wl.T * wl.H * 2
    for call in ROW_CALLS:
        diff = meas[call]["bytes"] - model[call]
        # the row kernels: within 2.5 % (measured 1.000 to 1.021 on the
        # large layers) ...
        lo = hi = max(0.025 * model[call], slack)
        if lists and call in ("dispatch", "combine_bwd"):
            # ... except token rows fetched again by the list walk: at most
            # two more reads of the token matrix (measured 1.2 and 1.7)
            hi = max(hi, 2 * token_bytes)
        assert -lo <= diff <= hi, (wname, call, diff / model[call])
    # the route's two passes hand the packed slot ranks and the per-block
    # counts through memory, and a dense route writes its row list (8 bytes
    # per row), none of which the model counts: measured 1.10 to 1.24 times
    # the model without the list, 1.36 to 1.41 with it, a few MB at most
    r = meas["route"]["bytes"] / model["route"]
    extra = 8 * wl.T * min(wl.k, wl.num_local) if lists else 0
    assert 1.0 <= r and meas["route"]["bytes"] <= 1.3 * model["route"] + extra + slack, (wname, r)


def test_dispatch_combine_pair():
    """us_per_layer.dispatch_combine: the two calls' algorithmic bytes over
    their summed device time, as a fraction of the 8 TB/s peak."""
    k = {"dispatch": {"avg_us": 200.0, "alg_bytes": 1.2e9},
         "combine": {"avg_us": 200.0, "alg_bytes": 1.2e9}}
    r = bench.dispatch_combine(k)
    assert r == {"us": 400.0, "GBps": 6000.0, "frac": 0.75}


def test_traffic_is_null_once_sources_change(monkeypatch):
    t = traffic()
    w = next(iter(t["workloads"]))
    if t["source_sha256"] == bench.kernel_source_sha256():
        assert bench.measured_traffic(w, "combine_bwd") == int(t["workloads"][w]["combine_bwd"]["bytes"])
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: "0" * 64)
    assert bench.measured_traffic(w, "combine_bwd") is None


def test_cpu_baseline_single_and_all_cores():
    """The oracle leg on a tiny layer, with host tensors standing in for the
    device buffers: one thread in-process, then one oracle per core in child
    processes that read the same arrays memory-mapped."""
    import torch

    wl = inputs.WORKLOADS["tiny"]
    idx, w = inputs.make_routing(wl, 1001)
    R = wl.T * wl.k
    gen = torch.Generator().manual_seed(5)
    st = {"idx_np": idx, "w_np": w}
    for n, rows in (("x", wl.T), ("g", wl.T), ("Y", R), ("F", R)):
        st[n] = torch.randn((rows, wl.H), generator=gen).to(torch.bfloat16)
    out = bench.cpu_baseline(wl, st, 0.3, torch)
    assert out["kind"] == "oracle" and out["cores"] == 1 and out["value"] > 0
    allc = out["all_cores"]
    assert allc["cores"] == bench.host_cores() and allc["processes"] == allc["cores"]
    assert allc["value"] > 0 and "processes" in allc["sample"]
