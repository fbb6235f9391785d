"""The route's row list against the token walk, on the GPU.

For dense routing the route also writes a (row, token) list into the handle's
workspace, and moe_dispatch and moe_combine_bwd walk that list instead of the
tokens when the handle brings the workspace.  Every case below routes once
and then runs both walks along the same handle tensors (one handle with the
workspace, one without):
  - the list holds each data row's (row, token) pair exactly once and no
    other pair (the workspace is filled with -1 before the route);
  - rows, row weights, row tokens and experts, and grad rows (with and
    without dw) agree bit for bit between the walks and with the oracle; dw
    of both walks meets the oracle's bar (exact products, fp64 sums, one
    rounding);
  - a list with two tokens exchanged moves exactly those two rows, so the
    list is what the dispatch follows when the handle brings it;
  - moe_route_dispatch over the list: eager rows past the total are left as
    they were, sync-free rows equal the token walk's;
  - the sync-free route, the list dispatch and the list combine backward
    captured in one HIP graph and replayed on new inputs, with eager work in
    between, equal the same calls run eagerly.
The cases cover tiles on every XCD and fewer route blocks than XCDs, a ragged
last tile, padding, sync-free sentinel rows, repeated and out-of-range ids,
k > EL, a local share of the experts, rows whose length is not a whole number
of the kernel's 4 KiB batches, and a route with no data row.
"""
import dataclasses
import zlib

import numpy as np
import pytest
import torch

import oracle
from combine_topk_idx_multihot_amd import binding as B
from combine_topk_idx_multihot_amd import inputs
from test_gpu_parity import check_dw, gpu, say, to_dev_bf16, to_np_u16  # noqa: F401 (gpu: fixture)

pytestmark = pytest.mark.gpu

CASES = [
    # (label, T, E, k, lb, EL, P, sync_free, H, p_invalid, dup, bad)
    ("tiles_on_every_xcd", 3000, 64, 8, 0, 64, 1, False, 512, 0.05, False, False),
    ("ragged_tail_padded", 1027, 16, 4, 0, 16, 3, False, 768, 0.1, False, False),
    ("sync_free_sentinels", 999, 32, 6, 0, 32, 5, True, 1280, 0.2, False, False),
    ("dups_and_bad_ids", 2000, 12, 5, 0, 12, 2, False, 256, 0.1, True, True),
    ("k_gt_EL", 1500, 8, 8, 3, 2, 2, False, 256, 0.05, True, False),
    ("fewer_blocks_than_xcds", 300, 16, 8, 0, 16, 4, True, 512, 0.05, False, False),
    ("half_the_experts_local", 2048, 64, 8, 16, 32, 1, False, 2304, 0.0, False, False),
    ("wide_rows", 1200, 8, 2, 0, 8, 1, False, 9216, 0.0, False, False),
    ("no_data_row", 1200, 8, 2, 0, 8, 4, False, 256, 1.0, False, False),
]


def _up256(n):
    return (n + 255) // 256 * 256


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


def list_offset(T, k, EL):
    """Byte offset of the row list in the workspace: after the route's
    per-block counts and flags, each 256-byte aligned."""
    nblk = route_blocks(T, k, EL)
    return _up256(nblk * EL * 4) + _up256(nblk * 4)


def has_list(T, E, k, EL):
    nblk = route_blocks(T, k, EL)
    return nblk > 1 and nblk * EL <= 65536 and k * EL >= 2 * E


def token_walk(h):
    """The same handle tensors without the workspace: the row kernels walk tokens."""
    return dataclasses.replace(h, workspace=None)


def list_pairs(h, T, k, EL):
    ws = h.workspace.cpu().numpy()
    return ws[list_offset(T, k, EL):].view(np.int32).reshape(-1, 2)


def make(case):
    label, T, E, k, lb, EL, P, sync_free, H, p_inv, dup, bad = case
    rng = np.random.default_rng(zlib.crc32(("row-list " + label).encode()))
    idx = inputs.random_routing(T, E, k, rng, p_invalid=p_inv, allow_dup=dup,
                                p_out_of_range=0.1 if bad else 0.0)
    w = rng.random((T, k), dtype=np.float32)
    x = inputs.bf16_normal((T, H), rng)
    g = inputs.bf16_normal((T, H), rng)
    C = oracle.capacity_min(T, k, EL, P) + (5 if sync_free else 0)
    d = B.make_desc(T, k, E, lb, EL, P, B.MOE_SYNC_FREE if sync_free else B.MOE_EAGER, False,
                    C if sync_free else 0)
    return rng, idx, w, x, g, C, d


def route(d, idx, bad):
    h = B.alloc_handle(d)
    h.workspace.fill_(-1)
    try:
        B.moe_route_build(d, torch.from_numpy(idx.astype(np.int32)).cuda(), h)
        assert not bad or d.mode == B.MOE_SYNC_FREE
    except B.MoeError as e:
        assert bad and e.code == B.MOE_ERR_INDEX, (e.code, B.last_error())
    torch.cuda.synchronize()
    return h


def walk(d, h, R, x_t, w_t, g_t, F_t):
    rows, row_w, rt, re = B.dispatch(d, h, x_t, w_t)
    gr, dw = B.combine_bwd(d, h, g_t, R, F_t)
    torch.cuda.synchronize()
    return dict(rows=to_np_u16(rows), row_w=row_w.cpu().numpy().view(np.uint32),
                row_token=rt.cpu().numpy(), row_expert=re.cpu().numpy(),
                grad_rows=to_np_u16(gr), dw=dw.cpu().numpy())


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_list_walk_matches_token_walk_and_oracle(case):
    label, T, E, k, lb, EL, P, sync_free, H, p_inv, dup, bad = case
    say(f"[row list] {label} T={T} E={E} k={k} lb={lb} EL={EL} P={P} sync_free={sync_free} H={H}")
    assert has_list(T, E, k, EL)
    rng, idx, w, x, g, C, d = make(case)
    ref = oracle.route(idx, E, lb, EL, P, sync_free=sync_free, C=C, w=w, x=x)
    h = route(d, idx, bad)
    R = C if sync_free else int(h.host_status[0])
    assert R == ref.R
    np.testing.assert_array_equal(h.row_of_slot.cpu().numpy(), ref.row_of_slot)

    # the list: each data row's (row, token) once, nothing else
    pairs = list_pairs(h, T, k, EL)
    got = pairs[pairs[:, 0] >= 0]
    data = np.flatnonzero(ref.row_token >= 0)
    assert len(got) == len(data)
    order = np.argsort(got[:, 0], kind="stable")
    np.testing.assert_array_equal(got[order, 0], data)
    np.testing.assert_array_equal(got[order, 1], ref.row_token[data])
    assert (pairs[pairs[:, 0] < 0] == -1).all()

    F = inputs.bf16_normal((R, H), rng)
    x_t, w_t, g_t = to_dev_bf16(x), torch.from_numpy(w).cuda(), to_dev_bf16(g)
    F_t = to_dev_bf16(F)  # empty when R = 0: dw is still written (zeros)
    by_list = walk(d, h, R, x_t, w_t, g_t, F_t)
    by_token = walk(d, token_walk(h), R, x_t, w_t, g_t, F_t)
    for key in ("rows", "row_w", "row_token", "row_expert", "grad_rows"):
        np.testing.assert_array_equal(by_list[key], by_token[key], err_msg=key)
    np.testing.assert_array_equal(by_list["row_token"], ref.row_token)
    np.testing.assert_array_equal(by_list["row_expert"], ref.row_expert)
    np.testing.assert_array_equal(by_list["row_w"], ref.row_w.view(np.uint32))
    np.testing.assert_array_equal(by_list["rows"], ref.rows)
    gr, dw = oracle.combine_bwd(idx, ref.row_of_slot, ref.row_token, g, E, lb, EL, F=F, R=R)
    np.testing.assert_array_equal(by_list["grad_rows"], gr)
    for res in (by_list, by_token):
        check_dw(res["dw"], dw, idx, ref.row_of_slot, g, F, lb, EL, E)
    # the combine backward without expert outputs (grad rows only, no dw)
    for hh in (h, token_walk(h)):
        gr_only, no_dw = B.combine_bwd(d, hh, g_t, R)
        torch.cuda.synchronize()
        assert no_dw is None
        np.testing.assert_array_equal(to_np_u16(gr_only), gr)


def test_dispatch_follows_the_list():
    """Two list entries of one route block with their tokens exchanged: the
    list walk writes each of those rows from the other token and every other
    row as the token walk does."""
    case = CASES[0]
    label, T, E, k, lb, EL, P, sync_free, H = case[:9]
    say(f"[row list] exchanged tokens, {label}")
    rng, idx, w, x, g, C, d = make(case)
    h = route(d, idx, False)
    per = 512 // k
    pairs = list_pairs(h, T, k, EL)
    valid = np.flatnonzero(pairs[:, 0] >= 0)
    tok = pairs[valid, 1]
    # the first two entries whose tokens differ but share a route block
    i1 = i2 = None
    for a in range(len(valid)):
        same = np.flatnonzero((tok // per == tok[a] // per) & (tok != tok[a]))
        if len(same):
            i1, i2 = valid[a], valid[same[0]]
            break
    assert i1 is not None
    (r1, t1), (r2, t2) = pairs[i1].tolist(), pairs[i2].tolist()
    off = list_offset(T, k, EL) // 4
    words = h.workspace.view(torch.int32)
    words[off + 2 * i1 + 1] = t2
    words[off + 2 * i2 + 1] = t1
    x_t = to_dev_bf16(x)
    rows_l = to_np_u16(B.dispatch(d, h, x_t)[0])
    rows_t = to_np_u16(B.dispatch(d, token_walk(h), x_t)[0])
    np.testing.assert_array_equal(rows_l[r1], x[t2])
    np.testing.assert_array_equal(rows_l[r2], x[t1])
    keep = np.ones(len(rows_l), bool)
    keep[[r1, r2]] = False
    np.testing.assert_array_equal(rows_l[keep], rows_t[keep])


@pytest.mark.parametrize("sync_free", [False, True], ids=["eager", "sync_free"])
def test_route_dispatch_over_the_list(sync_free):
    """moe_route_dispatch with a workspace (the list walk) against
    moe_dispatch along a handle without one (the token walk): eager rows
    [0, total) equal and rows past the total untouched; sync-free rows all
    equal."""
    case = ("route_dispatch", 4096, 128, 8, 0, 128, 16, sync_free, 1024, 0.05, True, False)
    label, T, E, k, lb, EL, P, _, H = case[:9]
    say(f"[row list] moe_route_dispatch sync_free={sync_free} T={T} E={E} k={k} P={P} H={H}")
    assert has_list(T, E, k, EL)
    rng, idx, w, x, g, C, d = make(case)
    R_cap = C if sync_free else oracle.capacity_min(T, k, EL, P)
    x_t, w_t = to_dev_bf16(x), torch.from_numpy(w).cuda()
    h = B.alloc_handle(d)
    rows = torch.full((R_cap, H), 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    row_w = torch.full((R_cap,), -7.0, dtype=torch.float32, device="cuda")
    rt = torch.full((R_cap,), -9, dtype=torch.int32, device="cuda")
    re = torch.full((R_cap,), -9, dtype=torch.int32, device="cuda")
    B.moe_route_dispatch(d, torch.from_numpy(idx.astype(np.int32)).cuda(), h, x_t, H, rows, w_t,
                         None, row_w, rt, re)
    torch.cuda.synchronize()
    R = C if sync_free else int(h.host_status[0])
    ref_rows, ref_w, ref_t, ref_e = B.dispatch(d, token_walk(h), x_t, w_t)
    torch.cuda.synchronize()
    rows_np = to_np_u16(rows)
    np.testing.assert_array_equal(rows_np[:R], to_np_u16(ref_rows))
    np.testing.assert_array_equal(row_w[:R].cpu().numpy().view(np.uint32),
                                  ref_w.cpu().numpy().view(np.uint32))
    np.testing.assert_array_equal(rt[:R].cpu().numpy(), ref_t.cpu().numpy())
    np.testing.assert_array_equal(re[:R].cpu().numpy(), ref_e.cpu().numpy())
    assert (rows_np[R:] == 0x5A5A).all()
    assert (row_w[R:].cpu().numpy() == -7.0).all()
    assert (rt[R:].cpu().numpy() == -9).all() and (re[R:].cpu().numpy() == -9).all()
    ref = oracle.route(idx, E, lb, EL, P, sync_free=sync_free, C=C, w=w, x=x)
    np.testing.assert_array_equal(rows_np[:R], ref.rows)


def test_list_walks_replay_from_a_graph():
    """Sync-free route (writing the list) + dispatch + combine backward with dw
    captured in one HIP graph; each replay, on ids, tokens and gradients copied
    into the captured buffers, equals an eager run of the same calls (also
    with the list) on the same inputs."""
    T, E, k, EL, P, H = 2048, 64, 8, 64, 4, 512
    assert has_list(T, E, k, EL)
    C = oracle.capacity_min(T, k, EL, P)
    d = B.make_desc(T, k, E, 0, EL, P, B.MOE_SYNC_FREE, False, C)
    say(f"[row list] graph replays T={T} E={E} k={k} EL={EL} P={P} H={H} C={C}")

    def inputs_(seed):
        r = np.random.default_rng(seed)
        return (inputs.random_routing(T, E, k, r, p_invalid=0.05, allow_dup=True).astype(np.int32),
                r.random((T, k), dtype=np.float32), inputs.bf16_normal((T, H), r),
                inputs.bf16_normal((T, H), r), inputs.bf16_normal((C, H), r))

    idx0, w0, x0, g0, F0 = inputs_(1)
    idx_t, w_t = torch.from_numpy(idx0).cuda(), torch.from_numpy(w0).cuda()
    x_t, g_t, F_t = to_dev_bf16(x0), to_dev_bf16(g0), to_dev_bf16(F0)
    h = B.alloc_handle(d)
    rows = torch.empty((C, H), dtype=torch.bfloat16, device="cuda")
    row_w = torch.empty(C, dtype=torch.float32, device="cuda")
    rt = torch.empty(C, dtype=torch.int32, device="cuda")
    re = torch.empty(C, dtype=torch.int32, device="cuda")
    gr = torch.empty((C, H), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()

    def step():
        B.moe_route_build(d, idx_t, h, stream=stream)
        B.moe_dispatch(d, h, x_t, H, C, rows, w_t, row_w, rt, re, stream=stream)
        B.moe_combine_bwd(d, h, g_t, H, C, gr, F_t, dw, stream=stream)

    with torch.cuda.stream(stream):
        step()  # warm-up outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step()
    torch.cuda.synchronize()
    for seed in (2, 3, 4):
        idx, w, x, g, F = inputs_(seed)
        idx_t.copy_(torch.from_numpy(idx))
        w_t.copy_(torch.from_numpy(w))
        x_t.copy_(to_dev_bf16(x))
        g_t.copy_(to_dev_bf16(g))
        F_t.copy_(to_dev_bf16(F))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (to_np_u16(rows), row_w.cpu().numpy().view(np.uint32), rt.cpu().numpy(),
               re.cpu().numpy(), to_np_u16(gr), dw.cpu().numpy().view(np.uint32))
        # the same calls eagerly on fresh outputs (eager work between replays)
        with torch.cuda.stream(stream):
            step()
        torch.cuda.synchronize()
        want = (to_np_u16(rows), row_w.cpu().numpy().view(np.uint32), rt.cpu().numpy(),
                re.cpu().numpy(), to_np_u16(gr), dw.cpu().numpy().view(np.uint32))
        for name, a_, b_ in zip(("rows", "row_w", "row_token", "row_expert", "grad_rows", "dw"),
                                got, want):
            np.testing.assert_array_equal(a_, b_, err_msg=f"replay seed {seed}: {name}")
        ref = oracle.route(idx, E, 0, EL, P, sync_free=True, C=C, w=w, x=x)
        np.testing.assert_array_equal(got[0], ref.rows)
        np.testing.assert_array_equal(got[2], ref.row_token)
