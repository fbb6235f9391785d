"""moe_route_dispatch on the GPU: the eager route and dispatch in one call,
with the dispatch queued before the row count is read back.

It is held against moe_route_build followed by moe_dispatch with R = total.
These must match bit for bit: the handle's metadata, the host status, the
multihot probs, and rows [0, total) of every dispatch output.  Rows at or past
the total must keep what the buffers held before.  The cases cover pinned and
pageable host status, ragged and padded routing, out-of-range ids (the call
returns MOE_ERR_INDEX after the readback, and the dispatch has run with those
slots empty), one token, and no tokens.
"""
import numpy as np
import pytest
import torch

from combine_topk_idx_multihot_amd import binding as B
from combine_topk_idx_multihot_amd import inputs
import oracle
from test_gpu_parity import gpu, say, to_dev_bf16, to_np_u16  # noqa: F401 (gpu: fixture)

pytestmark = pytest.mark.gpu

CASES = [
    # (label, T, E, k, lb, EL, P, H, p_invalid, p_bad, pinned)
    ("qwen_like", 4096, 128, 8, 0, 128, 16, 2048, 0.0, 0.0, True),
    ("ragged_padded", 1027, 40, 6, 4, 30, 7, 768, 0.1, 0.0, True),
    ("pageable_status", 999, 32, 4, 0, 32, 3, 512, 0.05, 0.0, False),
    ("bad_ids", 500, 16, 4, 0, 16, 2, 256, 0.1, 0.05, True),
    ("one_token", 1, 8, 4, 2, 5, 4, 256, 0.0, 0.0, True),
    ("no_tokens", 0, 8, 2, 0, 8, 4, 256, 0.0, 0.0, True),
    # the route's three-launch form (516 route blocks x 128 local experts)
    ("large_route", 33000, 128, 8, 0, 128, 16, 256, 0.02, 0.0, True),
]


def handle_for(d, pinned):
    h = B.alloc_handle(d)
    if not pinned:
        h = B.Handle(desc=d, routing_map=h.routing_map, tokens_per_expert=h.tokens_per_expert,
                     padded_offsets=h.padded_offsets, row_of_slot=h.row_of_slot, status=h.status,
                     host_status=torch.zeros(4, dtype=torch.int32), workspace=h.workspace)
    return h


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_route_dispatch_matches_two_calls(case):
    label, T, E, k, lb, EL, P, H, p_inv, p_bad, pinned = case
    say(f"[route_dispatch] {label} T={T} E={E} k={k} lb={lb} EL={EL} P={P} H={H} pinned={pinned}")
    rng = np.random.default_rng([31, T, E, k, EL, P])
    idx = inputs.random_routing(T, E, k, rng, p_invalid=p_inv, p_out_of_range=p_bad)
    d = B.make_desc(T, k, E, lb, EL, P, B.MOE_EAGER, False, 0)
    cap = B.moe_capacity_min(d)
    idx_t = torch.from_numpy(idx.astype(np.int32)).cuda()
    w = torch.rand((T, k), device="cuda")
    x = torch.randn((T, H), device="cuda").to(torch.bfloat16)

    # reference: the two calls
    h1 = handle_for(d, pinned)
    probs1 = torch.empty((T, E), dtype=torch.float32, device="cuda")
    rc1 = B.MOE_OK
    try:
        B.moe_route_build(d, idx_t, h1, w, probs1)
    except B.MoeError as e:
        rc1 = e.code
    R = int(h1.host_status[0])
    ref = B.dispatch(d, h1, x, w)
    torch.cuda.synchronize()

    # one call, into buffers of the worst case holding a marker
    h2 = handle_for(d, pinned)
    probs2 = torch.empty((T, E), dtype=torch.float32, device="cuda")
    rows = torch.full((cap, H), -3.0, dtype=torch.bfloat16, device="cuda")
    row_w = torch.full((cap,), -5.0, device="cuda")
    rt = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    re = torch.full((cap,), -9, dtype=torch.int32, device="cuda")
    rc2 = B.MOE_OK
    try:
        B.moe_route_dispatch(d, idx_t, h2, x, H, rows, w, probs2, row_w, rt, re)
    except B.MoeError as e:
        rc2 = e.code
    torch.cuda.synchronize()

    assert rc1 == rc2 == (B.MOE_ERR_INDEX if p_bad > 0 else B.MOE_OK)
    assert h2.host_status.tolist()[:3] == h1.host_status.tolist()[:3]
    assert int(h2.host_status[0]) == R
    for name in ("routing_map", "tokens_per_expert", "padded_offsets", "row_of_slot", "status"):
        assert torch.equal(getattr(h1, name), getattr(h2, name)), name
    assert torch.equal(probs1.view(torch.int32), probs2.view(torch.int32))
    assert torch.equal(rows[:R], ref[0])
    assert torch.equal(row_w[:R].view(torch.int32), ref[1].view(torch.int32))
    assert torch.equal(rt[:R], ref[2])
    assert torch.equal(re[:R], ref[3])
    # rows past the total are not written
    assert bool((rows[R:] == -3.0).all()) and bool((row_w[R:] == -5.0).all())
    assert bool((rt[R:] == -7).all()) and bool((re[R:] == -9).all())
    say(f"  total={R} of {cap} rows")


def test_route_dispatch_timed_and_repeated():
    """The call under a timing request spans the route and the dispatch, and
    repeated calls through one handle give the same rows every time."""
    T, E, k, P, H = 2048, 64, 8, 16, 1024
    rng = np.random.default_rng(5)
    idx = inputs.random_routing(T, E, k, rng)
    d = B.make_desc(T, k, E, 0, E, P, B.MOE_EAGER, False, 0)
    cap = B.moe_capacity_min(d)
    h = B.alloc_handle(d)
    idx_t = torch.from_numpy(idx.astype(np.int32)).cuda()
    w = torch.rand((T, k), device="cuda")
    x = torch.randn((T, H), device="cuda").to(torch.bfloat16)
    rows = torch.empty((cap, H), dtype=torch.bfloat16, device="cuda")
    row_w = torch.empty(cap, device="cuda")
    B.moe_route_dispatch(d, idx_t, h, x, H, rows, w, None, row_w)
    R = h.total
    first = rows[:R].clone()
    timer = B.KernelTimer()
    torch.cuda.synchronize()
    for i in range(5):
        if i == 2:
            timer.arm()
        B.moe_route_dispatch(d, idx_t, h, x, H, rows, w, None, row_w)
        assert h.total == R
    torch.cuda.synchronize()
    assert torch.equal(rows[:R], first)
    ms = timer.elapsed_ms()
    say(f"[route_dispatch] timed call: {ms * 1e3:.1f} us (route and dispatch)")
    assert 0.0 < ms < 10.0


SYNC_FREE_CASES = [
    # (label, T, E, k, lb, EL, P, H, p_invalid, p_bad, dup, idx64): T*k <= 16 runs the route in
    # the dispatch's own launch; the others take the route's and the dispatch's launches
    ("sf_decode_t1", 1, 128, 8, 0, 32, 1, 2048, 0.0, 0.0, False, False),
    ("sf_decode_t1_h4096", 1, 128, 8, 32, 32, 1, 4096, 0.0, 0.0, False, False),
    ("sf_t2_k8_padded", 2, 128, 8, 0, 128, 16, 512, 0.1, 0.0, False, False),
    ("sf_t1_k16_dups_bad", 1, 40, 16, 4, 30, 2, 768, 0.1, 0.1, True, False),
    ("sf_t3_k5_ragged_dups", 3, 20, 5, 2, 15, 3, 256, 0.1, 0.05, True, False),
    ("sf_t16_k1_int64", 16, 12, 1, 0, 12, 5, 256, 0.2, 0.0, False, True),
    ("sf_t2_many_local", 2, 1024, 8, 0, 1024, 2, 256, 0.0, 0.0, False, False),
    ("sf_t1_all_invalid", 1, 8, 4, 0, 8, 4, 256, 1.0, 0.0, False, False),
    ("sf_t17_k1_two_launches", 17, 64, 1, 0, 64, 1, 256, 0.0, 0.0, False, False),
    ("sf_t8_k8_two_launches", 8, 128, 8, 0, 32, 1, 512, 0.0, 0.0, False, False),
    ("sf_t1_k64_two_launches", 1, 100, 64, 10, 80, 3, 256, 0.05, 0.0, True, False),
    ("sf_t300_two_launches", 300, 64, 6, 8, 40, 3, 256, 0.05, 0.05, True, False),
    ("sf_no_tokens", 0, 8, 2, 0, 8, 4, 256, 0.0, 0.0, False, False),
]


@pytest.mark.parametrize("case", SYNC_FREE_CASES, ids=[c[0] for c in SYNC_FREE_CASES])
@pytest.mark.parametrize("meta", [True, False], ids=["meta", "rows_only"])
def test_sync_free_route_dispatch_matches_two_calls(case, meta):
    """Sync-free moe_route_dispatch (one launch for decode-sized routes)
    against moe_route_build + moe_dispatch: the handle, the probs and every
    one of the capacity's rows, bit for bit, and the oracle's route."""
    label, T, E, k, lb, EL, P, H, p_inv, p_bad, dup, idx64 = case
    say(f"[route_dispatch sync-free] {label} meta={meta}")
    rng = np.random.default_rng([37, T, E, k, EL, P])
    idx = inputs.random_routing(T, E, k, rng, p_invalid=p_inv, p_out_of_range=p_bad,
                                allow_dup=dup)
    C = B.moe_capacity_min(B.make_desc(T, k, E, lb, EL, P)) + 3
    d = B.make_desc(T, k, E, lb, EL, P, B.MOE_SYNC_FREE, idx64, C)
    idx_t = torch.from_numpy(idx.astype(np.int64 if idx64 else np.int32)).cuda()
    w = torch.rand((T, k), device="cuda")
    x = torch.randn((T, H), device="cuda").to(torch.bfloat16)

    h1 = B.alloc_handle(d)
    probs1 = torch.empty((T, E), dtype=torch.float32, device="cuda") if meta else None
    B.moe_route_build(d, idx_t, h1, w if meta else None, probs1)
    ref = B.dispatch(d, h1, x, w if meta else None, meta=meta)
    torch.cuda.synchronize()

    h2 = B.alloc_handle(d)
    for t in (h2.routing_map, h2.tokens_per_expert, h2.padded_offsets, h2.row_of_slot, h2.status):
        t.fill_(0x5A)  # a word the call fails to write shows up
    probs2 = torch.full((T, E), float("nan"), device="cuda") if meta else None
    rows = torch.full((C, H), -3.0, dtype=torch.bfloat16, device="cuda")
    row_w = torch.full((C,), -5.0, device="cuda") if meta else None
    rt = torch.full((C,), -7, dtype=torch.int32, device="cuda") if meta else None
    re = torch.full((C,), -9, dtype=torch.int32, device="cuda") if meta else None
    B.moe_route_dispatch(d, idx_t, h2, x, H, rows, w if meta else None, probs2, row_w, rt, re)
    torch.cuda.synchronize()
    for name in ("routing_map", "tokens_per_expert", "padded_offsets", "row_of_slot", "status"):
        assert torch.equal(getattr(h1, name), getattr(h2, name)), name
    assert torch.equal(rows.view(torch.int16), ref[0].view(torch.int16))
    if meta:
        assert torch.equal(probs1.view(torch.int32), probs2.view(torch.int32))
        for got, want in zip((row_w, rt, re), ref[1:]):
            assert torch.equal(got.view(torch.int32), want.view(torch.int32))
    # and the oracle's route
    o = oracle.route(idx, E, lb, EL, P, sync_free=True, C=C)
    np.testing.assert_array_equal(h2.row_of_slot.cpu().numpy(), o.row_of_slot)
    np.testing.assert_array_equal(h2.padded_offsets.cpu().numpy(), o.off)
    assert int(h2.status[0]) == o.total and int(h2.status[1]) & 3 == o.flags


def test_sync_free_route_dispatch_graph_replays():
    """The one-launch decode route and dispatch captured in a HIP graph with a
    combine after it, replayed on new ids and tokens copied into the captured
    buffers: every replay equals the two-call path on the same inputs."""
    T, E, k, EL, H = 4, 128, 8, 32, 1024
    C = B.moe_capacity_min(B.make_desc(T, k, E, 0, EL, 1))
    d = B.make_desc(T, k, E, 0, EL, 1, B.MOE_SYNC_FREE, False, C)
    idx_t = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((T, k), device="cuda")
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    h = B.alloc_handle(d)
    rows = torch.empty((C, H), dtype=torch.bfloat16, device="cuda")
    row_w = torch.empty(C, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def layer(s):
        B.moe_route_dispatch(d, idx_t, h, x, H, rows, w, None, row_w, stream=s)
        B.moe_combine(d, h, rows, H, C, out, stream=s)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        g.capture_begin()
        layer(s)
        g.capture_end()
    torch.cuda.synchronize()
    for rep in range(4):
        rng = np.random.default_rng([38, rep])
        idx = inputs.random_routing(T, E, k, rng, p_invalid=0.1)
        idx_t.copy_(torch.from_numpy(idx.astype(np.int32)))
        w.copy_(torch.rand((T, k)))
        x.copy_(torch.randn((T, H)).to(torch.bfloat16))
        rows.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        h1, _ = B.route(d, idx_t)
        r1 = B.dispatch(d, h1, x, w, meta=False)
        o1 = B.combine(d, h1, r1[0])
        torch.cuda.synchronize()
        say(f"[route_dispatch graph] replay {rep}")
        assert torch.equal(h.row_of_slot, h1.row_of_slot)
        assert torch.equal(rows.view(torch.int16), r1[0].view(torch.int16))
        assert torch.equal(row_w.view(torch.int32), r1[1].view(torch.int32))
        assert torch.equal(out.view(torch.int16), o1.view(torch.int16))


EAGER_WORKLOADS = [n for n, wl in inputs.WORKLOADS.items() if not wl.sync_free]


@pytest.mark.parametrize("name", EAGER_WORKLOADS)
def test_route_dispatch_full_size_against_oracle(name):
    """The call the benchmark times for eager layers, at the layer's full size
    and into its worst-case buffers, held directly against the oracle."""
    wl = inputs.WORKLOADS[name]
    say(f"[route_dispatch] full size vs oracle: {name} T={wl.T} H={wl.H} E={wl.E} k={wl.k} "
        f"P={wl.P}")
    case = inputs.make_case(wl)
    ref = oracle.route(case.idx, wl.E, wl.lb, wl.num_local, wl.P, w=case.w, x=case.x,
                       want_probs=True)
    assert ref.rc == oracle.OK
    T, k, H = wl.T, wl.k, wl.H
    d = B.make_desc(T, k, wl.E, wl.lb, wl.num_local, wl.P, B.MOE_EAGER, False, 0)
    cap = B.moe_capacity_min(d)
    h = B.alloc_handle(d)
    idx_t = torch.from_numpy(np.ascontiguousarray(case.idx, np.int32)).cuda()
    w_t = torch.from_numpy(np.ascontiguousarray(case.w, np.float32)).cuda()
    probs = torch.empty((T, wl.E), dtype=torch.float32, device="cuda")
    rows = torch.empty((cap, H), dtype=torch.bfloat16, device="cuda")
    row_w = torch.empty(cap, device="cuda")
    rt = torch.empty(cap, dtype=torch.int32, device="cuda")
    re = torch.empty(cap, dtype=torch.int32, device="cuda")
    B.moe_route_dispatch(d, idx_t, h, to_dev_bf16(case.x), H, rows, w_t, probs, row_w, rt, re)
    torch.cuda.synchronize()
    R = h.total
    assert R == ref.total and h.flags == ref.flags
    np.testing.assert_array_equal(h.routing_map.cpu().numpy(), ref.map)
    np.testing.assert_array_equal(h.tokens_per_expert.cpu().numpy(), ref.tpe)
    np.testing.assert_array_equal(h.padded_offsets.cpu().numpy(), ref.off)
    np.testing.assert_array_equal(h.row_of_slot.cpu().numpy(), ref.row_of_slot)
    np.testing.assert_array_equal(probs.cpu().numpy().view(np.uint32), ref.probs.view(np.uint32))
    np.testing.assert_array_equal(to_np_u16(rows[:R]), ref.rows)
    np.testing.assert_array_equal(row_w[:R].cpu().numpy().view(np.uint32), ref.row_w.view(np.uint32))
    np.testing.assert_array_equal(rt[:R].cpu().numpy(), ref.row_token)
    np.testing.assert_array_equal(re[:R].cpu().numpy(), ref.row_expert)
    say(f"  total={R} of {cap} rows, bit-exact")
