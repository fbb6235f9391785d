"""GPU parity: the HIP library against the oracle, through the C ABI.

Every case runs route, dispatch, combine, the combine backward (with dw) and
the dispatch backward (grad_x and the routing-weight gradients).

Routing metadata, permutation, dispatched rows and weights are compared bit for
bit; combine is expected bit-exact too (same slot order, same rounding) and is
held at least to 1e-6 relative; dw (exact products, fp64 sums in a different
order, one rounding to fp32) is held to |dw - ref| <= 1e-6*|ref| + 1e-12*sum|g*f|.

Cases: the five workloads at full size (the launch configuration the benchmark
times) plus small edge cases (ragged token counts, empty and all-invalid
routing, repeated ids, bad ids, topk=1, one token, E not a multiple of 16,
more than 512 local experts, sync-free with T=0).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from combine_topk_idx_multihot_amd import binding as B
from combine_topk_idx_multihot_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.moe_device_check(0)
    yield


def to_dev_bf16(a_u16):
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).view(torch.bfloat16).cuda()


def to_np_u16(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def f32_of_bf16(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def say(msg):
    print(msg, flush=True)


class Run:
    """One pass of the whole path on the GPU, outputs copied back to numpy."""

    def __init__(self, idx, w, x, E, lb=0, EL=None, P=1, sync_free=False, C=0, idx64=False,
                 grad=None, F=None, want_probs=True, f32_out=False, Y=None):
        T, k = idx.shape
        EL = E if EL is None else EL
        self.desc = B.make_desc(T, k, E, lb, EL, P, B.MOE_SYNC_FREE if sync_free else B.MOE_EAGER,
                                idx64, C if sync_free else 0)
        d = self.desc
        idx_t = torch.from_numpy(np.ascontiguousarray(idx, np.int64 if idx64 else np.int32)).cuda()
        w_t = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
        x_t = to_dev_bf16(x)
        self.rc = B.MOE_OK
        h = B.alloc_handle(d)
        probs = torch.empty((T, E), dtype=torch.float32, device="cuda") if want_probs else None
        try:
            B.moe_route_build(d, idx_t, h, w_t if want_probs else None, probs)
        except B.MoeError as e:
            self.rc = e.code
        torch.cuda.synchronize()
        self.h = h
        self.status = h.status.cpu().numpy()
        R = C if sync_free else int(h.host_status[0])
        self.R = R
        rows, row_w, rt, re = B.dispatch(d, h, x_t, w_t)
        Yin = rows if Y is None else to_dev_bf16(Y)
        out = B.combine(d, h, Yin, out_dtype=torch.float32 if f32_out else torch.bfloat16)
        torch.cuda.synchronize()
        self.map = h.routing_map.cpu().numpy()
        self.tpe = h.tokens_per_expert.cpu().numpy()
        self.off = h.padded_offsets.cpu().numpy()
        self.row_of_slot = h.row_of_slot.cpu().numpy()
        self.probs = probs.cpu().numpy() if want_probs else None
        self.rows = to_np_u16(rows)
        self.row_w = row_w.cpu().numpy()
        self.row_token = rt.cpu().numpy()
        self.row_expert = re.cpu().numpy()
        self.out = out.cpu().numpy() if f32_out else to_np_u16(out)
        self.status_after = h.status.cpu().numpy()
        if grad is not None:
            g_t = to_dev_bf16(grad)
            F_t = to_dev_bf16(F) if F is not None else None
            gr, dw = B.combine_bwd(d, h, g_t, R, F_t)
            torch.cuda.synchronize()
            self.grad_rows = to_np_u16(gr)
            self.dw = dw.cpu().numpy() if dw is not None else None
        if F is not None:
            # dispatch backward of (grad rows = F, grad row weights = a ramp)
            self.grad_row_w = (np.arange(R, dtype=np.float32) * np.float32(0.001) - np.float32(3.0))
            gx, gtw = B.dispatch_bwd(d, h, to_dev_bf16(F), torch.from_numpy(self.grad_row_w).cuda(),
                                     out_dtype=torch.float32 if f32_out else torch.bfloat16)
            torch.cuda.synchronize()
            self.grad_x = gx.cpu().numpy() if f32_out else to_np_u16(gx)
            self.grad_topk_w = gtw.cpu().numpy()


def check_against_oracle(run, idx, w, x, E, lb=0, EL=None, P=1, sync_free=False, C=0, grad=None,
                         F=None, f32_out=False, Y=None, expect_rc=oracle.OK):
    EL = E if EL is None else EL
    ref = oracle.route(idx, E, lb, EL, P, sync_free=sync_free, C=C, w=w, x=x, want_probs=True)
    assert ref.rc == expect_rc
    # the library reports out-of-range ids through its return code in eager
    # mode only (after its one sync); sync-free calls leave it to flag bit 0
    lib_rc = oracle.OK if (sync_free and ref.rc == oracle.ERR_INDEX) else ref.rc
    assert run.rc == lib_rc, (run.rc, B.last_error())
    # routing metadata: bit-exact
    np.testing.assert_array_equal(run.map, ref.map)
    np.testing.assert_array_equal(run.probs.view(np.uint32), ref.probs.view(np.uint32))
    np.testing.assert_array_equal(run.tpe, ref.tpe)
    np.testing.assert_array_equal(run.off, ref.off)
    np.testing.assert_array_equal(run.row_of_slot, ref.row_of_slot)
    assert run.status[0] == ref.total
    assert run.status[1] & 3 == ref.flags
    assert run.status[2] == ref.tpe.sum()
    assert run.R == ref.R
    # dispatch: bit-exact rows, weights, tokens, experts
    np.testing.assert_array_equal(run.row_token, ref.row_token)
    np.testing.assert_array_equal(run.row_expert, ref.row_expert)
    np.testing.assert_array_equal(run.row_w.view(np.uint32), ref.row_w.view(np.uint32))
    np.testing.assert_array_equal(run.rows, ref.rows)
    # combine: expected bit-exact; floor 1e-6 relative
    Yr = ref.rows if Y is None else Y
    exp = oracle.combine(idx, ref.row_of_slot, Yr, E, lb, EL, out="f32" if f32_out else "bf16")
    if f32_out:
        np.testing.assert_allclose(run.out, exp, rtol=1e-6, atol=0)
        np.testing.assert_array_equal(run.out.view(np.uint32), exp.view(np.uint32))
    else:
        np.testing.assert_allclose(f32_of_bf16(run.out), f32_of_bf16(exp), rtol=1e-6, atol=0)
        np.testing.assert_array_equal(run.out, exp)
    if grad is not None:
        gr, dw = oracle.combine_bwd(idx, ref.row_of_slot, ref.row_token, grad, E, lb, EL, F=F, R=ref.R)
        np.testing.assert_array_equal(run.grad_rows, gr)
        if F is not None:
            check_dw(run.dw, dw, idx, ref.row_of_slot, grad, F, lb, EL, E)
    if F is not None:
        gx, gtw = oracle.dispatch_bwd(idx, ref.row_of_slot, F, E, lb, EL, grad_row_w=run.grad_row_w,
                                      out="f32" if f32_out else "bf16")
        np.testing.assert_array_equal(run.grad_x.view(np.uint32 if f32_out else np.uint16),
                                      gx.view(np.uint32 if f32_out else np.uint16))
        np.testing.assert_array_equal(run.grad_topk_w.view(np.uint32), gtw.view(np.uint32))


def check_dw(got, ref, idx, row_of_slot, g, F, lb, EL, E, chunk=1024):
    T, k = idx.shape
    gf = f32_of_bf16(g)
    Ff = f32_of_bf16(F)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        gc = gf[t0:t1].astype(np.float64)
        for j in range(k):
            r = row_of_slot[t0:t1, j]
            ok = r >= 0
            mass = np.zeros(t1 - t0)
            if ok.any():
                mass[ok] = np.abs(gc[ok] * Ff[r[ok]].astype(np.float64)).sum(1)
            tol = 1e-6 * np.abs(ref[t0:t1, j].astype(np.float64)) + 1e-12 * mass
            err = np.abs(got[t0:t1, j].astype(np.float64) - ref[t0:t1, j].astype(np.float64))
            assert (err <= tol).all(), (t0, j, err.max())
            assert (got[t0:t1, j][~ok] == 0).all()


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_parity(name):
    wl = inputs.WORKLOADS[name]
    say(f"[parity] workload={name} T={wl.T} H={wl.H} E={wl.E} k={wl.k} EL={wl.num_local} "
        f"P={wl.P} sync_free={wl.sync_free}")
    case = inputs.make_case(wl, grad=True)
    C = wl.cap if wl.sync_free else 0
    ref = oracle.route(case.idx, wl.E, wl.lb, wl.num_local, wl.P, sync_free=wl.sync_free, C=C)
    F = inputs.expert_out_rows(ref.R, wl.H, case.seed)
    run = Run(case.idx, case.w, case.x, wl.E, wl.lb, wl.num_local, wl.P, wl.sync_free, C,
              grad=case.grad_out, F=F)
    check_against_oracle(run, case.idx, case.w, case.x, wl.E, wl.lb, wl.num_local, wl.P,
                         wl.sync_free, C, grad=case.grad_out, F=F)


@pytest.mark.parametrize("name", ["qwen3_30b_a3b", "h4096_rank_share"])
def test_workload_parity_int64_idx_f32_out_expert_rows(name):
    wl = inputs.WORKLOADS[name]
    say(f"[parity] int64 idx + f32 combine of independent rows: {name}")
    case = inputs.make_case(wl, seed=77)
    C = wl.cap if wl.sync_free else 0
    ref = oracle.route(case.idx, wl.E, wl.lb, wl.num_local, wl.P, sync_free=wl.sync_free, C=C)
    Y = inputs.expert_out_rows(ref.R, wl.H, 78)
    run = Run(case.idx, case.w, case.x, wl.E, wl.lb, wl.num_local, wl.P, wl.sync_free, C,
              idx64=True, f32_out=True, Y=Y, F=Y)
    check_against_oracle(run, case.idx, case.w, case.x, wl.E, wl.lb, wl.num_local, wl.P,
                         wl.sync_free, C, f32_out=True, Y=Y, F=Y)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

EDGE = [
    # (label, T, E, k, lb, EL, P, sync_free, H, p_invalid, dup, bad)
    ("ragged_T", 1027, 16, 4, 0, 16, 3, False, 512, 0.1, False, False),
    ("ragged_sync_free", 999, 32, 6, 8, 12, 5, True, 768, 0.2, False, False),
    ("all_invalid", 300, 8, 2, 0, 8, 4, False, 256, 1.0, False, False),
    ("all_invalid_sync_free", 300, 8, 2, 0, 8, 4, True, 256, 1.0, False, False),
    ("duplicates", 513, 12, 5, 2, 7, 2, False, 256, 0.1, True, False),
    ("bad_ids", 200, 10, 3, 0, 10, 1, False, 256, 0.1, False, True),
    ("topk1", 700, 64, 1, 0, 64, 1, False, 1024, 0.0, False, False),
    ("single_token", 1, 8, 4, 0, 8, 8, False, 256, 0.0, False, False),
    ("single_token_sync_free", 1, 8, 4, 0, 8, 8, True, 256, 0.0, False, False),
    ("E_not_mult_16", 257, 13, 3, 1, 9, 2, False, 256, 0.1, False, False),
    ("many_local", 2048, 1024, 8, 0, 600, 4, False, 256, 0.05, False, False),
    ("k_not_dividing_1024", 1500, 96, 7, 0, 96, 16, False, 256, 0.05, False, False),
    ("big_H", 70, 8, 3, 0, 8, 2, False, 9216, 0.1, False, False),
    ("k_gt_EL", 400, 32, 8, 4, 3, 2, True, 256, 0.0, False, False),
    ("empty", 0, 8, 2, 0, 8, 4, False, 256, 0.0, False, False),
    ("empty_sync_free", 0, 8, 2, 0, 8, 4, True, 256, 0.0, False, False),
    ("max_local_1024", 700, 1024, 8, 0, 1024, 3, False, 256, 0.05, False, False),
    ("max_local_sync_free", 300, 1500, 6, 400, 1024, 2, True, 512, 0.05, False, False),
    ("max_k_64", 200, 100, 64, 10, 80, 2, False, 256, 0.05, False, False),
    ("max_k_64_sync_free", 100, 64, 64, 0, 64, 1, True, 256, 0.0, False, False),
    # the route in one counting workgroup: 512 slots at k = 8 (256 with more
    # than 512 local experts); up to 1024 slots in one 1024-thread workgroup
    # (EL <= 256), up to 2048 with 2 slots per thread (EL <= 64); one token
    # past each limit, and the expert limits on either side
    ("one_route_block", 64, 128, 8, 0, 128, 16, False, 512, 0.05, False, False),
    ("one_block_65_tokens", 65, 128, 8, 0, 128, 16, False, 512, 0.05, False, False),
    ("one_block_1024_slots", 128, 128, 8, 0, 128, 4, False, 256, 0.05, True, False),
    ("one_block_2048_slots", 256, 128, 8, 0, 64, 16, False, 512, 0.05, True, True),
    ("one_block_2048_slots_sync_free", 256, 128, 8, 0, 32, 1, True, 256, 0.1, True, False),
    ("one_block_k6_341_tokens", 341, 64, 6, 0, 64, 3, True, 256, 0.1, True, False),
    ("blocks_k6_342_tokens", 342, 64, 6, 0, 64, 3, True, 256, 0.1, True, False),
    ("blocks_257_tokens", 257, 128, 8, 0, 128, 16, False, 256, 0.05, False, False),
    ("one_block_256_local", 128, 512, 8, 0, 256, 2, False, 256, 0.05, False, False),
    ("blocks_257_local", 128, 512, 8, 0, 257, 2, False, 256, 0.05, False, False),
    ("one_block_64_local_2048_slots", 256, 256, 8, 0, 64, 2, True, 256, 0.05, True, False),
    ("blocks_65_local_2048_slots", 256, 256, 8, 0, 65, 2, True, 256, 0.05, True, False),
    ("one_route_block_sync_free", 64, 128, 8, 0, 32, 1, True, 512, 0.0, False, False),
    ("one_route_block_1024_local", 32, 1024, 8, 0, 1024, 2, True, 256, 0.05, True, False),
    ("two_route_blocks_1024_local", 33, 1024, 8, 0, 1024, 2, False, 256, 0.05, False, True),
    # sync-free row arrays on both sides of 32 MiB: the tail zeroed by the
    # rows' launch (16381 rows of 2 KiB) or by a launch of its own (16389)
    ("tail_in_rows_launch", 2047, 128, 8, 0, 16, 1, True, 1024, 0.0, False, False),
    ("tail_launch_of_its_own", 2048, 128, 8, 0, 16, 1, True, 1024, 0.0, False, False),
    # the route's three-launch form, taken when the count table (route blocks
    # x local experts) passes 65536 entries: 66 blocks x 1024 local experts;
    # 512 blocks x 128 (65536, the last fused-finish size) against 513 and
    # 516 blocks x 128; eager, sync-free, repeated and bad ids
    ("large_route_1024_local", 2100, 1024, 8, 0, 1024, 2, False, 256, 0.05, False, False),
    ("large_route_1024_local_sync_free", 2100, 1024, 8, 0, 1024, 2, True, 256, 0.05, False,
     False),
    ("fused_finish_at_limit", 32768, 128, 8, 0, 128, 16, False, 256, 0.02, False, False),
    ("large_route_past_limit", 32769, 128, 8, 0, 128, 16, False, 256, 0.02, False, False),
    ("large_route_128_local", 33000, 128, 8, 0, 128, 16, False, 256, 0.02, False, False),
    ("large_route_128_local_sync_free", 33000, 128, 8, 0, 128, 1, True, 256, 0.0, False, False),
    ("large_route_share_sync_free", 33000, 128, 8, 16, 16, 4, True, 256, 0.02, True, False),
    ("large_route_dups_bad_ids", 33000, 128, 8, 0, 128, 4, False, 256, 0.05, True, True),
    ("large_route_1024_local_132_blocks", 4200, 1024, 8, 0, 1024, 1, True, 256, 0.02, True,
     False),
    # an expert's pad rows shared by several workgroups (at most about 64 KiB
    # each): 99 rows of 4 KiB over 7, and 599 over the cap of 16, sync-free
    ("pad_slices_uneven", 300, 16, 4, 0, 16, 100, False, 2048, 0.1, False, False),
    ("pad_slices_capped_sync_free", 200, 8, 2, 0, 8, 600, True, 2048, 0.05, True, False),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge_parity(case):
    label, T, E, k, lb, EL, P, sync_free, H, p_inv, dup, bad = case
    say(f"[edge] {label} T={T} E={E} k={k} lb={lb} EL={EL} P={P} sync_free={sync_free} H={H}")
    # a seed fixed by the label (str hashes are salted per process)
    rng = np.random.default_rng(zlib.crc32(label.encode()))
    idx = inputs.random_routing(T, E, k, rng, p_invalid=p_inv, allow_dup=dup,
                                p_out_of_range=0.1 if bad else 0.0)
    w = rng.random((T, k), dtype=np.float32)
    x = inputs.bf16_normal((T, H), rng)
    g = inputs.bf16_normal((T, H), rng)
    C = oracle.capacity_min(T, k, EL, P) + (5 if sync_free else 0)
    ref = oracle.route(idx, E, lb, EL, P, sync_free=sync_free, C=C)
    F = inputs.bf16_normal((ref.R, H), rng)
    run = Run(idx, w, x, E, lb, EL, P, sync_free, C, grad=g, F=F)
    check_against_oracle(run, idx, w, x, E, lb, EL, P, sync_free, C, grad=g, F=F,
                         expect_rc=oracle.ERR_INDEX if (bad and not sync_free) else oracle.OK)


def test_sync_free_rows_equal_eager_prefix_and_sentinel_tail():
    wl = inputs.WORKLOADS["h4096_rank_share"]
    case = inputs.make_case(wl, seed=5)
    say("[sync-free vs eager] h4096_rank_share seed=5")
    sf = Run(case.idx, case.w, case.x, wl.E, wl.lb, wl.num_local, wl.P, True, wl.cap)
    eg = Run(case.idx, case.w, case.x, wl.E, wl.lb, wl.num_local, wl.P, False, 0)
    tot = eg.R
    assert sf.status[0] == tot
    np.testing.assert_array_equal(sf.rows[:tot], eg.rows)
    assert (sf.rows[tot:] == 0).all()
    assert (sf.row_expert[tot:] == wl.num_local).all() and (sf.row_token[tot:] == -1).all()
    np.testing.assert_array_equal(sf.out, eg.out)


def test_repeat_runs_are_bitwise_identical():
    wl = inputs.WORKLOADS["skewed"]
    case = inputs.make_case(wl, seed=11, grad=True)
    ref = oracle.route(case.idx, wl.E, wl.lb, wl.num_local, wl.P)
    F = inputs.expert_out_rows(ref.R, wl.H, 12)
    say("[determinism] skewed seed=11 twice")
    a = Run(case.idx, case.w, case.x, wl.E, P=wl.P, grad=case.grad_out, F=F)
    b = Run(case.idx, case.w, case.x, wl.E, P=wl.P, grad=case.grad_out, F=F)
    for name in ("map", "tpe", "off", "row_of_slot", "rows", "row_w", "row_token", "row_expert",
                 "out", "grad_rows", "dw"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name), err_msg=name)


def test_eager_rows_mismatch_flag():
    rng = np.random.default_rng(3)
    T, E, k, H = 64, 8, 2, 256
    idx = inputs.random_routing(T, E, k, rng)
    d = B.make_desc(T, k, E, pad_multiple=1)
    h, _ = B.route(d, torch.from_numpy(idx.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    total = h.total
    x = to_dev_bf16(inputs.bf16_normal((T, H), rng))
    R = total + 7  # larger than total: the tail becomes sentinel rows, flag bit 2
    rows = torch.full((R, H), 1.0, dtype=torch.bfloat16, device="cuda")
    re = torch.empty(R, dtype=torch.int32, device="cuda")
    B.moe_dispatch(d, h, x, H, R, rows, row_expert=re)
    torch.cuda.synchronize()
    assert int(h.status[1]) & B.MOE_FLAG_ROWS_MISMATCH
    assert (to_np_u16(rows[total:]) == 0).all()
    assert (re[total:].cpu().numpy() == E).all()


def test_graph_capture_replays_like_eager():
    """Sync-free route + dispatch + combine + combine_bwd captured in one HIP
    graph after an eager warm-up, replayed several times with eager work in
    between; every replay must equal the eager result."""
    wl = inputs.WORKLOADS["h4096_rank_share"]
    T, H = 2048, 1024
    rng = np.random.default_rng(21)
    idx = inputs.topk_softmax(T, wl.E, wl.k, rng)[0]
    w = rng.random((T, wl.k), dtype=np.float32)
    d = B.make_desc(T, wl.k, wl.E, 0, 16, 1, B.MOE_SYNC_FREE, False, T * 8)
    C = d.capacity
    idx_t = torch.from_numpy(idx).cuda()
    w_t = torch.from_numpy(w).cuda()
    x_t = to_dev_bf16(inputs.bf16_normal((T, H), rng))
    g_t = to_dev_bf16(inputs.bf16_normal((T, H), rng))
    F_t = to_dev_bf16(inputs.bf16_normal((C, H), rng))
    h = B.alloc_handle(d)
    rows = torch.empty((C, H), dtype=torch.bfloat16, device="cuda")
    row_w = torch.empty(C, dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    gr = torch.empty((C, H), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((T, wl.k), dtype=torch.float32, device="cuda")

    def step(stream=None):
        B.moe_route_build(d, idx_t, h, stream=stream)
        B.moe_dispatch(d, h, x_t, H, C, rows, w_t, row_w, stream=stream)
        B.moe_combine(d, h, rows, H, C, out, stream=stream)
        B.moe_combine_bwd(d, h, g_t, H, C, gr, F_t, dw, stream=stream)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (rows, row_w, out, gr, dw, h.row_of_slot)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step(s)  # warm-up on the capture stream
        torch.cuda.synchronize()
        graph.capture_begin()
        step(s)
        graph.capture_end()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (rows, out, gr, dw):
            t.zero_()
        h.row_of_slot.fill_(-5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((rows, row_w, out, gr, dw, h.row_of_slot), eager):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), rep
        _ = (x_t.float() * 2).sum().item()  # eager work between replays


def test_eager_readback_into_pageable_host_memory():
    """The row count also comes back when the caller's host status is pageable
    memory (the library copies it after the kernels instead of letting the
    kernel write it)."""
    rng = np.random.default_rng(8)
    T, E, k, P = 3000, 64, 6, 8
    idx = inputs.random_routing(T, E, k, rng, p_invalid=0.1)
    d = B.make_desc(T, k, E, pad_multiple=P)
    h = B.alloc_handle(d)
    h = B.Handle(desc=d, routing_map=h.routing_map, tokens_per_expert=h.tokens_per_expert,
                 padded_offsets=h.padded_offsets, row_of_slot=h.row_of_slot, status=h.status,
                 host_status=torch.full((4,), -9, dtype=torch.int32), workspace=h.workspace)
    assert not h.host_status.is_pinned()
    say("[pageable host status]")
    B.moe_route_build(d, torch.from_numpy(idx.astype(np.int32)).cuda(), h)
    ref = oracle.route(idx, E, P=P)
    assert list(h.host_status.numpy()[:3]) == [ref.total, ref.flags, int(ref.tpe.sum())]
    np.testing.assert_array_equal(h.row_of_slot.cpu().numpy(), ref.row_of_slot)


def test_two_streams_at_once():
    """Independent layers on two streams at the same time (the library keeps
    no state between calls): both match the oracle."""
    rng = np.random.default_rng(17)
    cases = []
    for i, (T, E, k, sf) in enumerate([(2000, 32, 4, True), (1500, 48, 6, False)]):
        idx = inputs.random_routing(T, E, k, rng, p_invalid=0.05)
        x = inputs.bf16_normal((T, 512), rng)
        w = rng.random((T, k), dtype=np.float32)
        C = oracle.capacity_min(T, k, E, 2) if sf else 0
        d = B.make_desc(T, k, E, 0, E, 2, B.MOE_SYNC_FREE if sf else B.MOE_EAGER, False, C)
        cases.append(dict(idx=idx, x=x, w=w, d=d, C=C, sf=sf, E=E, h=B.alloc_handle(d),
                          s=torch.cuda.Stream(), idx_t=torch.from_numpy(idx.astype(np.int32)).cuda(),
                          x_t=to_dev_bf16(x), w_t=torch.from_numpy(w).cuda()))
    torch.cuda.synchronize()
    say("[two streams]")
    outs = []
    for c in cases:  # both routes and dispatches queued before any result is read
        with torch.cuda.stream(c["s"]):
            B.moe_route_build(c["d"], c["idx_t"], c["h"], stream=c["s"])
            R = B.rows_for(c["d"], c["h"])
            rows, row_w, rt, re = B.dispatch(c["d"], c["h"], c["x_t"], c["w_t"], stream=c["s"])
            out = B.combine(c["d"], c["h"], rows, stream=c["s"])
            outs.append((rows, row_w, rt, out))
    torch.cuda.synchronize()
    for c, (rows, row_w, rt, out) in zip(cases, outs):
        ref = oracle.route(c["idx"], c["E"], P=2, sync_free=c["sf"], C=c["C"], w=c["w"], x=c["x"])
        np.testing.assert_array_equal(to_np_u16(rows), ref.rows)
        np.testing.assert_array_equal(rt.cpu().numpy(), ref.row_token)
        np.testing.assert_array_equal(row_w.cpu().numpy().view(np.uint32), ref.row_w.view(np.uint32))
        np.testing.assert_array_equal(to_np_u16(out), oracle.combine(c["idx"], ref.row_of_slot,
                                                                     ref.rows, c["E"]))


def test_nan_inf_and_poisoned_weights():
    """Non-finite data and poisoned weights: NaN payloads, infinities, -0 and
    subnormals are moved bit for bit; the weights of empty and non-local slots
    are NaN and must never reach a row; combine follows IEEE (bf16 output
    NaNs are the canonical 0x7FC0, fp32 output compared NaN for NaN)."""
    rng = np.random.default_rng(23)
    T, E, k, lb, EL, H = 400, 16, 4, 4, 8, 256
    idx = inputs.random_routing(T, E, k, rng, p_invalid=0.2)
    x = inputs.bf16_normal((T, H), rng)
    specials = np.array([0x7FC0, 0x7F81, 0xFFC1, 0x7F80, 0xFF80, 0x8000, 0x0001, 0x807F],
                        np.uint16)  # qNaN, sNaN-ish, -NaN, +inf, -inf, -0, subnormals
    pos = rng.random((T, H)) < 0.02
    x[pos] = rng.choice(specials, size=int(pos.sum()))
    w = rng.random((T, k), dtype=np.float32)
    local = (idx >= lb) & (idx < lb + EL)
    w[~local] = np.nan  # never to be read
    g = inputs.bf16_normal((T, H), rng)
    g[rng.random((T, H)) < 0.01] = 0x7F80
    say("[nan/inf] dispatch, combine (bf16 and fp32), combine_bwd")
    for f32_out in (False, True):
        run = Run(idx, w, x, E, lb, EL, 2, grad=g, F=None, want_probs=False, f32_out=f32_out)
        ref = oracle.route(idx, E, lb, EL, 2, w=w, x=x)
        np.testing.assert_array_equal(run.rows, ref.rows)                   # bits, NaNs included
        np.testing.assert_array_equal(run.row_w.view(np.uint32), ref.row_w.view(np.uint32))
        assert not np.isnan(run.row_w).any()
        exp = oracle.combine(idx, ref.row_of_slot, ref.rows, E, lb, EL, out="f32" if f32_out else "bf16")
        if f32_out:
            same = (run.out == exp) | (np.isnan(run.out) & np.isnan(exp))
            assert same.all()
        else:
            np.testing.assert_array_equal(run.out, exp)
        gr, _ = oracle.combine_bwd(idx, ref.row_of_slot, ref.row_token, g, E, lb, EL, R=ref.R)
        np.testing.assert_array_equal(run.grad_rows, gr)
