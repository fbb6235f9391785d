"""moe_time_next_call on the GPU: the library times one call's kernels into two
HIP events carried by the kernels' own dispatch packets.

Checked here:
- a timed call writes the same outputs, bit for bit, as an untimed one;
- its elapsed time is positive and no longer than that of events recorded on
  the stream around the call;
- the request covers one call only: a later untimed call, or a call that fails,
  leaves the events as they were;
- a sync-free call with two launches (tail fill, then rows) is timed from the
  first kernel's start to the last kernel's end;
- the binding's KernelTimer (events without the system-scope fence) times a
  call the same way.
"""
import numpy as np
import pytest
import torch

from combine_topk_idx_multihot_amd import binding as B
from combine_topk_idx_multihot_amd import inputs
from test_gpu_parity import gpu, say  # noqa: F401 (gpu: fixture)

pytestmark = pytest.mark.gpu


def events(n):
    s = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record(s)  # creates the HIP event
    torch.cuda.synchronize()
    return evs


def layer(T, H, E, k, EL, P, sync_free, seed):
    rng = np.random.default_rng(seed)
    idx = inputs.random_routing(T, E, k, rng, p_invalid=0.05)
    w = rng.random((T, k), dtype=np.float32)
    C = 0
    mode = B.MOE_SYNC_FREE if sync_free else B.MOE_EAGER
    d = B.make_desc(T, k, E, 0, EL, P, mode, False, 0)
    if sync_free:
        C = T * min(k, EL) + EL * (P - 1)
        d = B.make_desc(T, k, E, 0, EL, P, mode, False, C)
    idx_t = torch.from_numpy(idx.astype(np.int32)).cuda()
    w_t = torch.from_numpy(w).cuda()
    x = torch.randn((T, H), device="cuda").to(torch.bfloat16)
    h, _ = B.route(d, idx_t, w_t)
    torch.cuda.synchronize()
    return d, h, x, w_t


def same(a, b):
    return all(torch.equal(u, v) for u, v in zip(a, b))


def test_timed_call_matches_untimed_and_is_consumed():
    say("[timing] eager T=2048 H=1024 E=64 k=8")
    d, h, x, w = layer(2048, 1024, 64, 8, 64, 16, False, 1)
    s = torch.cuda.current_stream()
    ref = B.dispatch(d, h, x, w)
    got = tuple(torch.empty_like(t) for t in ref)
    torch.cuda.synchronize()
    e_in0, e_in1, e_out0, e_out1 = events(4)
    e_out0.record(s)
    B.moe_time_next_call(e_in0, e_in1)
    B.moe_dispatch(d, h, x, 1024, ref[0].shape[0], got[0], w, *got[1:])
    e_out1.record(s)
    torch.cuda.synchronize()
    assert same(ref, got)
    inner = e_in0.elapsed_time(e_in1)
    outer = e_out0.elapsed_time(e_out1)
    say(f"  kernel {inner * 1e3:.1f} us, stream events {outer * 1e3:.1f} us")
    assert 0.0 < inner <= outer * 1.01 + 2e-3

    # the request was used up: an untimed call leaves the events alone
    B.dispatch(d, h, x, w)
    B.combine(d, h, got[0])
    torch.cuda.synchronize()
    assert e_in0.elapsed_time(e_in1) == inner

    # a failing call drops the request as well
    B.moe_time_next_call(e_in0, e_in1)
    out = torch.empty((d.T, 1024), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.MoeError):
        B.moe_combine(d, h, got[0], 100, got[0].shape[0], out)
    B.combine(d, h, got[0])
    torch.cuda.synchronize()
    assert e_in0.elapsed_time(e_in1) == inner


def test_every_timed_entry_point():
    say("[timing] each entry point, eager T=1024 H=512 E=32 k=4")
    d, h, x, w = layer(1024, 512, 32, 4, 32, 4, False, 2)
    R = h.total
    ev = events(2)
    B.moe_time_next_call(*ev)
    rows, row_w, rt, re = B.dispatch(d, h, x, w)
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) > 0
    calls = {
        "route": lambda: B.route(d, torch.zeros((1024, 4), dtype=torch.int32, device="cuda"))[0],
        "dispatch_fp8": lambda: B.dispatch_fp8(d, h, x, w),
        "combine": lambda: B.combine(d, h, rows),
        "combine_bwd": lambda: B.combine_bwd(d, h, x, R, rows),
        "dispatch_bwd": lambda: B.dispatch_bwd(d, h, rows, row_w),
    }
    for name, call in calls.items():
        a, b = events(2)
        B.moe_time_next_call(a, b)
        call()
        torch.cuda.synchronize()
        t = a.elapsed_time(b)
        say(f"  {name}: {t * 1e3:.1f} us")
        assert t > 0, name


def test_sync_free_call_spans_tail_and_rows():
    # 8 of 64 experts local: the capacity (T*8 rows) is mostly tail, written
    # by the tail launch that precedes the rows' launch.  The call writes all
    # C*H*2 bytes of rows, which no kernel writes faster than the 8 TB/s HBM
    # peak; the rows' launch alone moves about a tenth of that.
    T, H = 8192, 2048
    say(f"[timing] sync-free T={T} H={H} E=64 EL=8 k=8")
    d, h, x, w = layer(T, H, 64, 8, 8, 1, True, 3)
    C = d.capacity
    s = torch.cuda.current_stream()
    rows = torch.empty((C, H), dtype=torch.bfloat16, device="cuda")
    row_w = torch.empty(C, dtype=torch.float32, device="cuda")
    B.moe_dispatch(d, h, x, H, C, rows, w, row_w)  # warm
    e_in0, e_in1, e_out0, e_out1 = events(4)
    e_out0.record(s)
    B.moe_time_next_call(e_in0, e_in1)
    B.moe_dispatch(d, h, x, H, C, rows, w, row_w)
    e_out1.record(s)
    torch.cuda.synchronize()
    inner = e_in0.elapsed_time(e_in1)
    outer = e_out0.elapsed_time(e_out1)
    floor_ms = C * H * 2 / 8e12 * 1e3
    say(f"  kernels {inner * 1e3:.1f} us, stream events {outer * 1e3:.1f} us, "
        f"write floor {floor_ms * 1e3:.1f} us")
    assert floor_ms <= inner <= outer * 1.01 + 2e-3


def test_kernel_timer():
    say("[timing] KernelTimer, eager T=2048 H=1024 E=64 k=8")
    d, h, x, w = layer(2048, 1024, 64, 8, 64, 16, False, 4)
    ref = B.dispatch(d, h, x, w)
    got = tuple(torch.empty_like(t) for t in ref)
    t = B.KernelTimer()
    torch.cuda.synchronize()
    t.arm()
    B.moe_dispatch(d, h, x, 1024, ref[0].shape[0], got[0], w, *got[1:])
    torch.cuda.synchronize()
    assert same(ref, got)
    ms = t.elapsed_ms()
    say(f"  dispatch {ms * 1e3:.1f} us")
    # a layer of this size moves ~80 MB: between 1 us and 10 ms
    assert 1e-3 < ms < 10.0
    t.close()
