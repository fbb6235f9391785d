"""GPU parity of the FP8 dispatch (moe_dispatch_fp8) against the oracle.

E4M3 codes, block scales, row weights, tokens and experts are compared bit
for bit.  Small cases compare every row; the full-size workloads compare a
seeded sample of data rows (the oracle quantizes a row by a plain scan of the
code table, too slow for a whole 16K x 4096 batch) and check on every row the
properties that hold at any size: non-data rows are zero codes with zero
scales, and all rows of one token are identical.
"""
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


def say(msg):
    print(msg, flush=True)


def to_dev_bf16(a_u16):
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_bits(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


class RunFp8:
    def __init__(self, idx, w, x, E, lb, EL, P, sync_free, C, idx64=False):
        T, k = idx.shape
        d = B.make_desc(T, k, E, lb, EL, P, B.MOE_SYNC_FREE if sync_free else B.MOE_EAGER, idx64,
                        C if sync_free else 0)
        h = B.alloc_handle(d)
        idx_t = torch.from_numpy(np.ascontiguousarray(idx, np.int64 if idx64 else np.int32)).cuda()
        self.rc = B.MOE_OK
        try:
            B.moe_route_build(d, idx_t, h)
        except B.MoeError as e:
            self.rc = e.code
        torch.cuda.synchronize()
        self.R = B.rows_for(d, h)
        q, s, rw, rt, re = B.dispatch_fp8(d, h, to_dev_bf16(x), torch.from_numpy(w).cuda())
        torch.cuda.synchronize()
        self.q = q.view(torch.uint8).cpu().numpy()
        self.s = s.cpu().numpy()
        self.row_w = rw.cpu().numpy()
        self.row_token = rt.cpu().numpy()
        self.row_expert = re.cpu().numpy()
        self.flags = int(h.status[1])


def check_meta(run, ref):
    assert run.R == ref.R
    np.testing.assert_array_equal(run.row_token, ref.row_token)
    np.testing.assert_array_equal(run.row_expert, ref.row_expert)
    np.testing.assert_array_equal(run.row_w.view(np.uint32), ref.row_w.view(np.uint32))


def check_all_rows(run, ref, x):
    q, s = oracle.dispatch_fp8(x, ref.row_token)
    np.testing.assert_array_equal(run.q, q)
    np.testing.assert_array_equal(run.s.view(np.uint32), s.view(np.uint32))


def check_sampled_rows(run, ref, x, n=48, seed=0):
    data = np.nonzero(ref.row_token >= 0)[0]
    rng = np.random.default_rng(seed)
    pick = np.unique(np.concatenate([rng.choice(data, min(n, data.size), replace=False),
                                     data[:2], data[-2:]])) if data.size else data
    q, s = oracle.dispatch_fp8(x, ref.row_token[pick])
    np.testing.assert_array_equal(run.q[pick], q)
    np.testing.assert_array_equal(run.s[pick].view(np.uint32), s.view(np.uint32))
    # every row: non-data rows are zero; rows of one token are equal
    other = ref.row_token < 0
    assert not run.q[other].any() and not run.s[other].any()
    first = np.full(x.shape[0], -1, np.int64)
    toks = ref.row_token[data]
    first[toks[::-1]] = data[::-1]  # lowest row of each token
    for c0 in range(0, data.size, 4096):
        r = data[c0:c0 + 4096]
        f = first[ref.row_token[r]]
        np.testing.assert_array_equal(run.q[r], run.q[f])
        np.testing.assert_array_equal(run.s[r], run.s[f])


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_fp8_workload(name):
    wl = inputs.WORKLOADS[name]
    say(f"[fp8] workload={name} T={wl.T} H={wl.H} E={wl.E} k={wl.k} EL={wl.num_local} P={wl.P} "
        f"sync_free={wl.sync_free}")
    case = inputs.make_case(wl)
    C = wl.cap if wl.sync_free else 0
    ref = oracle.route(case.idx, wl.E, wl.lb, wl.num_local, wl.P, sync_free=wl.sync_free, C=C,
                       w=case.w)
    run = RunFp8(case.idx, case.w, case.x, wl.E, wl.lb, wl.num_local, wl.P, wl.sync_free, C)
    assert run.rc == ref.rc == oracle.OK
    check_meta(run, ref)
    if wl.T * wl.H <= 1 << 21:
        check_all_rows(run, ref, case.x)
    else:
        check_sampled_rows(run, ref, case.x)


EDGE = [
    # (label, T, E, k, lb, EL, P, sync_free, H, p_invalid, dup)
    ("ragged_T", 1027, 16, 4, 0, 16, 3, False, 512, 0.1, False),
    ("ragged_sync_free_H768", 999, 32, 6, 8, 12, 5, True, 768, 0.2, False),
    ("pads_H256", 300, 8, 2, 0, 8, 7, False, 256, 0.1, False),
    ("all_invalid_sync_free", 300, 8, 2, 0, 8, 4, True, 256, 1.0, False),
    ("duplicates", 513, 12, 5, 2, 7, 2, False, 1280, 0.1, True),
    ("topk1", 700, 64, 1, 0, 64, 1, False, 1024, 0.0, False),
    ("single_token_sync_free", 1, 8, 4, 0, 8, 8, True, 256, 0.0, False),
    ("many_local", 2048, 1024, 8, 0, 600, 4, False, 256, 0.05, False),
    ("big_H", 70, 8, 3, 0, 8, 2, False, 9216, 0.1, False),
    ("empty", 0, 8, 2, 0, 8, 4, False, 256, 0.0, False),
    ("empty_sync_free", 0, 8, 2, 0, 8, 4, True, 512, 0.0, False),
    # pad rows of 2112 bytes (codes and scales), 99 per expert over 4 workgroups
    ("pad_slices", 300, 16, 4, 0, 16, 100, False, 2048, 0.1, False),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_fp8_edge(case):
    label, T, E, k, lb, EL, P, sync_free, H, p_inv, dup = case
    say(f"[fp8 edge] {label} T={T} E={E} k={k} lb={lb} EL={EL} P={P} sync_free={sync_free} H={H}")
    rng = np.random.default_rng(sum(map(ord, label)))
    idx = inputs.random_routing(T, E, k, rng, p_invalid=p_inv, allow_dup=dup)
    w = rng.random((T, k), dtype=np.float32)
    x = inputs.bf16_normal((T, H), rng)
    C = oracle.capacity_min(T, k, EL, P) + (5 if sync_free else 0)
    ref = oracle.route(idx, E, lb, EL, P, sync_free=sync_free, C=C, w=w)
    run = RunFp8(idx, w, x, E, lb, EL, P, sync_free, C, idx64=(T % 2 == 1))
    assert run.rc == ref.rc == oracle.OK
    check_meta(run, ref)
    check_all_rows(run, ref, x)


def test_fp8_special_values():
    """Blocks at the scale floor, huge and tiny magnitudes, bf16 subnormals,
    negative zeros, exact ties after scaling, and a block whose maximum is 448."""
    rng = np.random.default_rng(99)
    T, E, k, H = 64, 4, 2, 512
    xf = rng.standard_normal((T, H)).astype(np.float32)
    xf[0] = 0.0
    xf[1] = -0.0
    xf[2] = rng.normal(0, 1e-7, H)                   # below the 1e-4 floor
    xf[3] = rng.normal(0, 1e30, H)                   # huge
    xf[4] = rng.normal(0, 1e-30, H)                  # tiny, still above bf16's smallest normal
    xf[5] = rng.choice([1e-39, -2e-39, 3e-40], H)    # bf16 subnormals
    xf[6, :128] = np.linspace(-448, 448, 128)        # scale exactly 1
    xf[7, :128] = 1.0625                             # a tie at scale 1 (plus one 448)
    xf[7, 0] = 448.0
    xf[8] = rng.standard_normal(H) * 1e-3
    xf[8, ::128] = 1.0                               # one large value per block: subnormal codes
    xf[9, :] = -0.0
    xf[9, 5] = 3.0
    x = bf16_bits(xf)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    w = rng.random((T, k), dtype=np.float32)
    for sync_free in (False, True):
        say(f"[fp8 special] sync_free={sync_free}")
        C = oracle.capacity_min(T, k, E, 2) if sync_free else 0
        ref = oracle.route(idx, E, 0, E, 2, sync_free=sync_free, C=C, w=w)
        run = RunFp8(idx, w, x, E, 0, E, 2, sync_free, C)
        check_meta(run, ref)
        check_all_rows(run, ref, x)


def test_fp8_rows_dequantize_close_to_bf16_rows():
    """The FP8 rows against the bf16 dispatch of the same routing: each code
    times its scale is within half a 3-bit-mantissa step of the bf16 value."""
    wl = inputs.WORKLOADS["qwen3_30b_a3b"]
    case = inputs.make_case(wl, seed=3)
    say("[fp8 vs bf16 rows] qwen3_30b_a3b seed=3")
    d = B.make_desc(wl.T, wl.k, wl.E, wl.lb, wl.num_local, wl.P)
    h, _ = B.route(d, torch.from_numpy(case.idx.astype(np.int32)).cuda())
    x = to_dev_bf16(case.x)
    rows = B.dispatch(d, h, x, meta=False)[0]
    q, s = B.dispatch_fp8(d, h, x, meta=False)[:2]
    deq = q.float() * s.repeat_interleave(128, dim=1)
    ref = rows.float()
    err = (deq - ref).abs()
    bound = torch.maximum(ref.abs() * 2.0 ** -4, s.repeat_interleave(128, dim=1) * 2.0 ** -10)
    assert bool((err <= bound * (1 + 1e-5) + 1e-6 * ref.abs()).all())


def test_fp8_sync_free_graph_replays_match_oracle():
    """Sync-free route + FP8 dispatch captured once in a HIP graph, replayed on
    three new inputs copied into the captured buffers (eager work between
    replays); every replay is checked against the oracle row by row."""
    T, E, k, lb, EL, P, H = 1000, 64, 6, 8, 24, 4, 768
    C = oracle.capacity_min(T, k, EL, P) + 11
    d = B.make_desc(T, k, E, lb, EL, P, B.MOE_SYNC_FREE, False, C)
    dev = "cuda"
    idx_t = torch.zeros((T, k), dtype=torch.int32, device=dev)
    w_t = torch.zeros((T, k), dtype=torch.float32, device=dev)
    x_t = torch.zeros((T, H), dtype=torch.bfloat16, device=dev)
    h = B.alloc_handle(d)
    q = torch.empty((C, H), dtype=torch.uint8, device=dev)
    sc = torch.empty((C, H // 128), dtype=torch.float32, device=dev)
    rw = torch.empty(C, dtype=torch.float32, device=dev)
    rt = torch.empty(C, dtype=torch.int32, device=dev)
    re = torch.empty(C, dtype=torch.int32, device=dev)

    def case(seed):
        rng = np.random.default_rng(seed)
        idx = inputs.random_routing(T, E, k, rng, p_invalid=0.1, allow_dup=True)
        return idx, rng.random((T, k), dtype=np.float32), inputs.bf16_normal((T, H), rng)

    def load(c):
        idx_t.copy_(torch.from_numpy(c[0].astype(np.int32)))
        w_t.copy_(torch.from_numpy(c[1]))
        x_t.copy_(to_dev_bf16(c[2]))

    def step(stream):
        B.moe_route_build(d, idx_t, h, stream=stream)
        B.moe_dispatch_fp8(d, h, x_t, H, C, q, sc, w_t, rw, rt, re, stream=stream)

    load(case(0))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step(s)
        torch.cuda.synchronize()
        graph.capture_begin()
        step(s)
        graph.capture_end()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for seed in (1, 2, 3):
        say(f"[fp8 graph] replay seed={seed}")
        c = case(seed)
        load(c)
        q.fill_(0x55)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = oracle.route(c[0], E, lb, EL, P, sync_free=True, C=C, w=c[1])
        rq, rs = oracle.dispatch_fp8(c[2], ref.row_token)
        np.testing.assert_array_equal(q.cpu().numpy(), rq)
        np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint32), rs.view(np.uint32))
        np.testing.assert_array_equal(rt.cpu().numpy(), ref.row_token)
        np.testing.assert_array_equal(re.cpu().numpy(), ref.row_expert)
        np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), ref.row_w.view(np.uint32))
        _ = (x_t.float() * 2).sum().item()  # eager work between replays


def test_fp8_eager_rows_mismatch_flag():
    """Eager mode with R above the routed total: rows past the total become
    sentinel rows (zero codes, zero scales, expert EL) and flag bit 2 is set."""
    rng = np.random.default_rng(4)
    T, E, k, H = 64, 8, 2, 768
    idx = inputs.random_routing(T, E, k, rng)
    d = B.make_desc(T, k, E, pad_multiple=1)
    h, _ = B.route(d, torch.from_numpy(idx.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    total = h.total
    x = to_dev_bf16(inputs.bf16_normal((T, H), rng))
    R = total + 9
    q = torch.full((R, H), 0x55, dtype=torch.uint8, device="cuda")
    sc = torch.full((R, H // 128), 7.0, dtype=torch.float32, device="cuda")
    re = torch.empty(R, dtype=torch.int32, device="cuda")
    say("[fp8 eager mismatch]")
    B.moe_dispatch_fp8(d, h, x, H, R, q, sc, row_expert=re)
    torch.cuda.synchronize()
    assert int(h.status[1]) & B.MOE_FLAG_ROWS_MISMATCH
    assert not q[total:].any() and not sc[total:].any()
    assert (re[total:].cpu().numpy() == E).all()
    ref = oracle.route(idx, E)
    rq, rs = oracle.dispatch_fp8(to_np(x), ref.row_token)
    np.testing.assert_array_equal(q[:total].cpu().numpy(), rq)
    np.testing.assert_array_equal(sc[:total].cpu().numpy().view(np.uint32), rs.view(np.uint32))


def to_np(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
