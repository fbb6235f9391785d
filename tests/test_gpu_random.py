"""GPU parity on seeded random configurations: token counts, slot counts,
expert ranges, pad multiples, hidden sizes, both modes, both id widths,
empty slots, repeated ids and out-of-range ids, drawn from one master seed.

Every call of the path runs on each configuration (route, dispatch, combine,
combine backward with dw, dispatch backward, FP8 dispatch, and in eager mode
the one-call route and dispatch) and is compared with the oracle exactly as in
test_gpu_parity / test_gpu_fp8.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_topk_idx_multihot_amd import binding as B
from combine_topk_idx_multihot_amd import inputs
from test_gpu_fp8 import RunFp8, check_all_rows, check_meta, check_sampled_rows
from test_gpu_parity import (Run, check_against_oracle, gpu, say, to_dev_bf16,  # noqa: F401
                             to_np_u16)

pytestmark = pytest.mark.gpu

N_CASES = 24


def draw(i):
    rng = np.random.default_rng([20261202, i])
    E = int(rng.choice([1, 3, 8, 16, 37, 64, 128, 300]))
    dup = bool(rng.random() < 0.3)
    kmax = min(E, 16) if not dup else 16
    k = int(rng.integers(1, kmax + 1))
    if rng.random() < 0.1 and dup:
        k = int(rng.choice([24, 40, 64]))
    EL = int(rng.integers(1, E + 1))
    lb = int(rng.integers(0, E - EL + 1))
    T = int(rng.choice([0, 1, 2, 63, 100, 511, 777, 1500]))
    P = int(rng.choice([1, 2, 3, 16, 64, 130]))
    H = int(rng.choice([256, 512, 768, 1280, 2048]))
    sync_free = bool(rng.random() < 0.5)
    idx64 = bool(rng.random() < 0.5)
    p_inv = float(rng.choice([0.0, 0.05, 0.5, 1.0]))
    bad = bool(rng.random() < 0.15)
    extra = int(rng.integers(0, 50))
    return dict(E=E, k=k, EL=EL, lb=lb, T=T, P=P, H=H, sync_free=sync_free, idx64=idx64,
                p_inv=p_inv, dup=dup, bad=bad, extra=extra, seed=i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i):
    c = draw(i)
    say(f"[random {i}] {c}")
    rng = np.random.default_rng([7, i])
    T, E, k, lb, EL, P, H = c["T"], c["E"], c["k"], c["lb"], c["EL"], c["P"], c["H"]
    idx = inputs.random_routing(T, E, k, rng, p_invalid=c["p_inv"], allow_dup=c["dup"],
                                p_out_of_range=0.05 if c["bad"] else 0.0)
    w = rng.random((T, k), dtype=np.float32)
    x = inputs.bf16_normal((T, H), rng)
    g = inputs.bf16_normal((T, H), rng)
    sf = c["sync_free"]
    C = oracle.capacity_min(T, k, EL, P) + (c["extra"] if sf else 0)
    ref = oracle.route(idx, E, lb, EL, P, sync_free=sf, C=C)
    F = inputs.bf16_normal((ref.R, H), rng)
    # the oracle returns ERR_INDEX whenever an id lies outside [-1, E)
    expect = oracle.ERR_INDEX if ref.flags & oracle.FLAG_BAD_ID else oracle.OK
    run = Run(idx, w, x, E, lb, EL, P, sf, C, idx64=c["idx64"], grad=g, F=F)
    check_against_oracle(run, idx, w, x, E, lb, EL, P, sf, C, grad=g, F=F, expect_rc=expect)
    run8 = RunFp8(idx, w, x, E, lb, EL, P, sf, C, idx64=c["idx64"])
    ref8 = oracle.route(idx, E, lb, EL, P, sync_free=sf, C=C, w=w)
    check_meta(run8, ref8)
    if ref8.R * H <= 1 << 21:
        check_all_rows(run8, ref8, x)
    else:
        check_sampled_rows(run8, ref8, x, n=32, seed=i)
    if not sf:
        check_route_dispatch(idx, w, x, E, lb, EL, P, c["idx64"], expect)


def check_route_dispatch(idx, w, x, E, lb, EL, P, idx64, expect):
    """moe_route_dispatch (the eager route and dispatch in one call, into
    worst-case buffers) against the oracle: metadata, probs and rows [0, total)."""
    T, k = idx.shape
    H = x.shape[1]
    ref = oracle.route(idx, E, lb, EL, P, w=w, x=x, want_probs=True)
    d = B.make_desc(T, k, E, lb, EL, P, B.MOE_EAGER, idx64, 0)
    cap = B.moe_capacity_min(d)
    h = B.alloc_handle(d)
    idx_t = torch.from_numpy(np.ascontiguousarray(idx, np.int64 if idx64 else np.int32)).cuda()
    w_t = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    probs = torch.empty((T, E), dtype=torch.float32, device="cuda")
    rows = torch.empty((cap, H), dtype=torch.bfloat16, device="cuda")
    row_w = torch.empty(cap, device="cuda")
    rt = torch.empty(cap, dtype=torch.int32, device="cuda")
    re = torch.empty(cap, dtype=torch.int32, device="cuda")
    rc = B.MOE_OK
    try:
        B.moe_route_dispatch(d, idx_t, h, to_dev_bf16(x), H, rows, w_t, probs, row_w, rt, re)
    except B.MoeError as e:
        rc = e.code
    torch.cuda.synchronize()
    assert rc == expect
    R = h.total
    assert R == ref.total and (h.flags & 3) == (ref.flags & 3)
    np.testing.assert_array_equal(h.routing_map.cpu().numpy(), ref.map)
    np.testing.assert_array_equal(h.tokens_per_expert.cpu().numpy(), ref.tpe)
    np.testing.assert_array_equal(h.padded_offsets.cpu().numpy(), ref.off)
    np.testing.assert_array_equal(h.row_of_slot.cpu().numpy(), ref.row_of_slot)
    np.testing.assert_array_equal(probs.cpu().numpy().view(np.uint32), ref.probs.view(np.uint32))
    np.testing.assert_array_equal(to_np_u16(rows[:R]), ref.rows)
    np.testing.assert_array_equal(row_w[:R].cpu().numpy().view(np.uint32), ref.row_w.view(np.uint32))
    np.testing.assert_array_equal(rt[:R].cpu().numpy(), ref.row_token)
    np.testing.assert_array_equal(re[:R].cpu().numpy(), ref.row_expert)
