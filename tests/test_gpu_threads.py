"""Host threads on the GPU: two threads drive independent layers at the same
time, each on its own stream (ctypes releases the interpreter lock during the
library's calls, so both eager readback waits spin at once).  Every output
matches, bit for bit, the same layer run alone.  A timing request made in one
thread is taken by that thread's next call only: the other thread's calls in
the meantime leave the events alone.
"""
import threading

import numpy as np
import pytest
import torch

from combine_topk_idx_multihot_amd import binding as B
from combine_topk_idx_multihot_amd import inputs
from test_gpu_parity import gpu, say  # noqa: F401 (gpu: fixture)

pytestmark = pytest.mark.gpu

ITERS = 12


def make_layer(T, H, E, k, P, sync_free, seed):
    rng = np.random.default_rng(seed)
    idx = inputs.random_routing(T, E, k, rng, p_invalid=0.05)
    C = T * min(k, E) + E * (P - 1) if sync_free else 0
    d = B.make_desc(T, k, E, 0, E, P, B.MOE_SYNC_FREE if sync_free else B.MOE_EAGER, False, C)
    return dict(d=d, h=B.alloc_handle(d), idx=torch.from_numpy(idx.astype(np.int32)).cuda(),
                w=torch.rand((T, k), device="cuda"),
                x=torch.randn((T, H), device="cuda").to(torch.bfloat16),
                g=torch.randn((T, H), device="cuda").to(torch.bfloat16))


def run_layer(c, stream, iters, timer=None):
    """`iters` passes of the whole path; the outputs of the last one."""
    d, h = c["d"], c["h"]
    with torch.cuda.stream(stream):
        for i in range(iters):
            if timer is not None and i == iters // 2:
                timer.arm()
            B.moe_route_build(d, c["idx"], h, stream=stream)
            R = B.rows_for(d, h)
            rows, row_w, rt, re = B.dispatch(d, h, c["x"], c["w"], stream=stream)
            out = B.combine(d, h, rows, stream=stream)
            grad_rows, dw = B.combine_bwd(d, h, c["g"], R, rows, stream=stream)
        stream.synchronize()
    return [rows, row_w, rt, re, out, grad_rows, dw]


def test_two_threads_two_streams():
    layers = [make_layer(3000, 1024, 64, 8, 16, False, 1), make_layer(2500, 768, 40, 6, 4, True, 2),
              make_layer(2000, 512, 32, 4, 1, False, 3)]
    streams = [torch.cuda.Stream() for _ in layers]
    say("[threads] serial references")
    refs = [run_layer(c, s, 1) for c, s in zip(layers, streams)]
    torch.cuda.synchronize()

    timer = B.KernelTimer()
    torch.cuda.synchronize()
    got = [None] * len(layers)
    errors = []

    def work(i):
        try:
            got[i] = run_layer(layers[i], streams[i], ITERS, timer if i == 0 else None)
        except Exception as e:  # reported below, in the main thread
            errors.append((i, repr(e)))

    say(f"[threads] {len(layers)} threads x {ITERS} passes")
    ts = [threading.Thread(target=work, args=(i,)) for i in range(len(layers))]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in ts), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(refs, got)):
        for j, (u, v) in enumerate(zip(a, b)):
            assert torch.equal(u, v), (i, j)
    ms = timer.elapsed_ms()
    say(f"  thread 0's timed route: {ms * 1e3:.1f} us")
    # the timed call was thread 0's route of a 3000-token layer: a few µs to
    # a few hundred, never the whole run of every thread
    assert 0.0 < ms < 5.0
