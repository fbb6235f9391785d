"""Pins for the oracle (CPU only).

The pages print no worked example, so each part of the oracle is pinned to
something that is not the oracle's own formula: a library routine that computes
the same thing another way (numpy fancy indexing, bincount, lexsort, argsort,
torch's bf16 conversion, float64 dot products), a closed form (combine of an
identity expert is k_valid * x; dw of an identity expert is <g, x>), an
invariant (sum of tokens_per_expert equals the number of valid local routes;
the adjoint identity between combine and its backward), a hand-derived example
(tests/golden/hand_example.json), or an exact bound.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from combine_topk_idx_multihot_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# helpers that compute expected values another way (library routines)
# --------------------------------------------------------------------------

def f32_of_bf16(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def torch_bf16(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def distinct_local_pairs(idx, E, lb, EL):
    """Set of (t, e) with a valid id e in the local range, via numpy only."""
    T, k = idx.shape
    t = np.repeat(np.arange(T), k)
    e = idx.reshape(-1)
    keep = (e >= lb) & (e < lb + EL) & (e < E)
    pairs = np.unique(np.stack([t[keep], e[keep]], 1), axis=0) if keep.any() else np.zeros((0, 2), int)
    return pairs


def expected_map(idx, E):
    T, k = idx.shape
    m = np.zeros((T, E), np.uint8)
    valid = (idx >= 0) & (idx < E)
    rows = np.repeat(np.arange(T)[:, None], k, 1)
    m[rows[valid], idx[valid]] = 1  # fancy-index assignment
    return m


def check_route_against_library(idx, E, lb, EL, P, r, sync_free=False, C=0, w=None):
    T, k = idx.shape
    # routing map: numpy fancy-index assignment
    np.testing.assert_array_equal(r.map, expected_map(idx, E))
    pairs = distinct_local_pairs(idx, E, lb, EL)
    # tokens_per_expert: bincount over distinct local (t, e) pairs
    tpe = np.bincount(pairs[:, 1] - lb, minlength=EL) if len(pairs) else np.zeros(EL, int)
    np.testing.assert_array_equal(r.tpe, tpe)
    assert r.tpe.sum() == len(pairs)  # invariant: sum = valid local routes
    # padded offsets: closed form cumsum(ceil(tpe/P)*P)
    off = np.concatenate([[0], np.cumsum(-(-tpe // P) * P)])
    np.testing.assert_array_equal(r.off, off)
    assert r.total == off[-1]
    R = C if sync_free else r.total
    assert r.R == R
    # data rows taken in order equal a library sort of (expert, token)
    is_data = r.row_token >= 0
    data_tok = r.row_token[is_data]
    data_exp = r.row_expert[is_data]
    order = np.lexsort((pairs[:, 0], pairs[:, 1])) if len(pairs) else np.zeros(0, int)
    np.testing.assert_array_equal(data_exp, pairs[order, 1] - lb)
    np.testing.assert_array_equal(data_tok, pairs[order, 0])
    # each expert's data rows start at its padded offset; the rest of its group
    # is pad (token -1, same expert); rows past total are the sentinel EL
    for e in range(EL):
        grp = slice(off[e], off[e + 1])
        assert (r.row_expert[grp] == e).all()
        assert (r.row_token[off[e]:off[e] + tpe[e]] >= 0).all()
        assert (r.row_token[off[e] + tpe[e]:off[e + 1]] == -1).all()
    assert (r.row_expert[r.total:R] == EL).all()
    assert (r.row_token[r.total:R] == -1).all()
    # row_of_slot: bijection with the data rows; -1 for invalid/non-local
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            row = r.row_of_slot[t, j]
            if lb <= e < lb + EL and e < E:
                assert r.row_token[row] == t and r.row_expert[row] == e - lb
            else:
                assert row == -1
    if w is not None:
        # distinct ids: row weight is the slot weight, bit for bit; repeated
        # ids: the float32 sum of the repeated slots' weights in slot order
        for t in range(T):
            seen = {}
            for j in range(k):
                e = idx[t, j]
                if lb <= e < lb + EL and e < E:
                    seen.setdefault(e, []).append(np.float32(w[t, j]))
            for e, ws in seen.items():
                acc = ws[0]
                for v in ws[1:]:
                    acc = np.float32(acc + v)
                row = r.row_of_slot[t, list(idx[t]).index(e)]
                assert r.row_w[row].view(np.uint32) == np.float32(acc).view(np.uint32)
        assert (r.row_w[r.row_token < 0] == 0).all()


# --------------------------------------------------------------------------
# bf16 rounding (used by combine's bf16 output)
# --------------------------------------------------------------------------

def test_bf16_round_matches_torch_on_bit_sweep():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    special = []
    for hi in (0x0000, 0x0001, 0x007F, 0x0080, 0x3F80, 0x3F81, 0x7F7E, 0x7F7F, 0x7F80):
        for lo in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF):
            for s in (0, 0x80000000):
                special.append(s | (hi << 16) | lo)
    bits = np.concatenate([bits, np.array(special, np.uint32)])
    f = bits.view(np.float32)
    ours = oracle.bf16_round(f)
    nan = np.isnan(f)
    np.testing.assert_array_equal(ours[~nan], torch_bf16(f[~nan]))
    assert (ours[nan] == 0x7FC0).all()


def test_bf16_round_tie_and_overflow_cases():
    # 1 + 2^-8 is halfway between 1 and 1+2^-7: ties to even -> 1.0 (0x3F80)
    assert oracle.bf16_round([1.0 + 2.0 ** -8])[0] == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even) -> 0x3F82
    assert oracle.bf16_round([1.0 + 3 * 2.0 ** -8])[0] == 0x3F82
    # the midpoint between the largest finite bf16 and 2^128 overflows to inf
    mid = np.array([0x7F7F8000], np.uint32).view(np.float32)
    assert oracle.bf16_round(mid)[0] == 0x7F80
    below = np.array([0x7F7F7FFF], np.uint32).view(np.float32)
    assert oracle.bf16_round(below)[0] == 0x7F7F
    assert oracle.bf16_round([-0.0])[0] == 0x8000


# --------------------------------------------------------------------------
# hand-derived worked example
# --------------------------------------------------------------------------

def test_hand_example():
    with open(os.path.join(GOLDEN, "hand_example.json")) as fh:
        g = json.load(fh)
    idx = np.array(g["idx"])
    r = oracle.route(idx, E=g["E"], lb=g["lb"], EL=g["EL"], P=g["P"])
    assert r.rc == oracle.OK
    np.testing.assert_array_equal(r.tpe, g["tokens_per_expert"])
    np.testing.assert_array_equal(r.off, g["padded_offsets"])
    assert r.total == g["total"]
    np.testing.assert_array_equal(r.row_token, g["row_token"])
    np.testing.assert_array_equal(r.row_expert, g["row_expert"])
    np.testing.assert_array_equal(r.row_of_slot, g["row_of_slot"])
    assert oracle.capacity_min(len(idx), idx.shape[1], g["EL"], g["P"]) == g["sync_free_capacity_min"]
    rs = oracle.route(idx, E=g["E"], lb=g["lb"], EL=g["EL"], P=g["P"], sync_free=True,
                      C=g["sync_free_capacity_min"])
    np.testing.assert_array_equal(rs.row_expert, g["sync_free_row_expert"])
    np.testing.assert_array_equal(rs.row_token, g["sync_free_row_token"])
    # identity experts: combine(dispatch(x)) = k_valid * x
    x = inputs.bf16_normal((len(idx), 256), np.random.default_rng(3))
    rr = oracle.route(idx, E=g["E"], lb=g["lb"], EL=g["EL"], P=g["P"], x=x)
    out = oracle.combine(idx, rr.row_of_slot, rr.rows, E=g["E"], out="f32")
    kv = np.array(g["k_valid"], np.float32)[:, None]
    np.testing.assert_array_equal(out, f32_of_bf16(x) * kv)


# --------------------------------------------------------------------------
# routing metadata against library routines, many random tiny cases
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(40))
def test_route_random_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(0, 40))
    E = int(rng.integers(1, 12))
    k = int(rng.integers(1, min(E, 6) + 1))
    EL = int(rng.integers(1, E + 1))
    lb = int(rng.integers(0, E - EL + 1))
    P = int(rng.choice([1, 2, 3, 4, 8]))
    dup = bool(seed % 3 == 0)
    idx = inputs.random_routing(T, E, k, rng, p_invalid=0.25, allow_dup=dup)
    w = rng.random((T, k), dtype=np.float32)
    r = oracle.route(idx, E, lb, EL, P, w=w, want_probs=True)
    assert r.rc == oracle.OK
    check_route_against_library(idx, E, lb, EL, P, r, w=w)
    if not dup:
        assert r.flags & oracle.FLAG_DUP == 0
    # multihot probs: weight at the routed experts (sum over repeats), 0 elsewhere
    exp = np.zeros((T, E), np.float32)
    for t in range(T):
        seen = set()
        for j in range(k):
            e = idx[t, j]
            if 0 <= e < E:
                exp[t, e] = np.float32(exp[t, e] + w[t, j]) if e in seen else w[t, j]
                seen.add(e)
    np.testing.assert_allclose(r.probs, exp, rtol=0, atol=0)
    # sync-free at the minimum capacity: same data rows, zero sentinel tail
    C = oracle.capacity_min(T, k, EL, P)
    x = inputs.bf16_normal((T, 256), rng)
    re_ = oracle.route(idx, E, lb, EL, P, w=w, x=x)
    rs = oracle.route(idx, E, lb, EL, P, sync_free=True, C=C, w=w, x=x)
    check_route_against_library(idx, E, lb, EL, P, rs, sync_free=True, C=C, w=w)
    np.testing.assert_array_equal(rs.row_token[:r.total], r.row_token)
    np.testing.assert_array_equal(rs.row_of_slot, r.row_of_slot)
    np.testing.assert_array_equal(rs.rows[:r.total], re_.rows)
    data = re_.row_token >= 0
    np.testing.assert_array_equal(re_.rows[data], x[re_.row_token[data]])
    assert not re_.rows[~data].any()                   # pad rows: bf16 +0
    assert not rs.rows[r.total:].any()                 # sentinel rows: bf16 +0
    assert (rs.row_token[r.total:] == -1).all() and (rs.row_expert[r.total:] == EL).all()
    assert not rs.row_w[r.total:].any()


def test_top1_all_local_is_stable_argsort_and_combine_inverts():
    rng = np.random.default_rng(5)
    T, E = 300, 16
    idx = rng.integers(0, E, size=(T, 1))
    x = inputs.bf16_normal((T, 512), rng)
    r = oracle.route(idx, E, P=1, x=x)
    np.testing.assert_array_equal(r.row_token, np.argsort(idx[:, 0], kind="stable"))
    np.testing.assert_array_equal(r.rows, x[np.argsort(idx[:, 0], kind="stable")])
    out = oracle.combine(idx, r.row_of_slot, r.rows, E)
    np.testing.assert_array_equal(out, x)  # bit-for-bit round trip


# --------------------------------------------------------------------------
# combine: closed forms, order, bounds
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_combine_identity_experts_closed_form(seed):
    rng = np.random.default_rng(200 + seed)
    T, E, k, H = 64, 10, 4, 256
    EL, lb = (E, 0) if seed % 2 == 0 else (6, 3)
    idx = inputs.random_routing(T, E, k, rng, p_invalid=0.3, allow_dup=(seed % 3 == 1))
    x = inputs.bf16_normal((T, H), rng)
    r = oracle.route(idx, E, lb, EL, P=2 + seed % 3, x=x)
    kv = np.array([len({e for e in row if lb <= e < lb + EL}) for row in idx], np.float32)
    xf = f32_of_bf16(x)
    out32 = oracle.combine(idx, r.row_of_slot, r.rows, E, lb, EL, out="f32")
    # k_valid * x is exact in fp32 for k_valid <= 8 (and so is every partial
    # sum); a token with no local slot gives +0, not 0 * x (which may be -0)
    expect = np.where(kv[:, None] == 0, np.float32(0), xf * kv[:, None])
    np.testing.assert_array_equal(out32.view(np.uint32), expect.view(np.uint32))
    outbf = oracle.combine(idx, r.row_of_slot, r.rows, E, lb, EL, out="bf16")
    np.testing.assert_array_equal(outbf, torch_bf16(expect))
    # tokens with no local slot give +0 (bit pattern 0)
    assert (outbf[kv == 0] == 0).all()


def test_combine_adds_in_ascending_slot_order():
    # terms 2^30, -2^30, 1 in slots 0,1,2: ascending order gives 1; any order
    # adding 1 before the cancellation would give 0 (2^30 + 1 rounds to 2^30)
    idx = np.array([[0, 1, 2]])
    rows_f = np.array([[2.0 ** 30], [-(2.0 ** 30)], [1.0]], np.float32).repeat(256, 1)
    Y = torch_bf16(rows_f)
    r = oracle.route(idx, 3)
    Yperm = np.zeros_like(Y)
    for j in range(3):
        Yperm[r.row_of_slot[0, j]] = Y[j]
    out = oracle.combine(idx, r.row_of_slot, Yperm, 3, out="f32")
    assert (out == 1.0).all()
    idx2 = np.array([[0, 2, 1]])  # slot order 2^30, 1, -2^30 -> 0
    r2 = oracle.route(idx2, 3)
    Y2 = np.zeros_like(Y)
    for j, src in enumerate([0, 2, 1]):
        Y2[r2.row_of_slot[0, j]] = Y[src]
    out2 = oracle.combine(idx2, r2.row_of_slot, Y2, 3, out="f32")
    assert (out2 == 0.0).all()


def test_combine_negative_zero_and_single_slot_round_trip():
    idx = np.array([[1, -1], [-1, -1]])
    x = np.array([[0x8000] * 256, [0x3F80] * 256], np.uint16)  # -0.0 and 1.0
    r = oracle.route(idx, 2, x=x)
    out = oracle.combine(idx, r.row_of_slot, r.rows, 2)
    assert (out[0] == 0x8000).all()  # accumulator starts from the first term
    assert (out[1] == 0x0000).all()  # no local slot -> +0


@pytest.mark.parametrize("seed", range(4))
def test_combine_random_rows_within_fp32_bound(seed):
    rng = np.random.default_rng(300 + seed)
    T, E, k, H = 50, 8, 8, 256
    idx = inputs.random_routing(T, E, k, rng, p_invalid=0.2)
    r = oracle.route(idx, E, P=4)
    Y = inputs.bf16_normal((r.R, H), rng)
    out = oracle.combine(idx, r.row_of_slot, Y, E, out="f32").astype(np.float64)
    Yf = f32_of_bf16(Y).astype(np.float64)
    exact = np.zeros((T, H))
    mass = np.zeros((T, H))
    n = np.zeros(T)
    for t in range(T):
        for j in range(k):
            if idx[t, j] >= 0:
                exact[t] += Yf[r.row_of_slot[t, j]]
                mass[t] += np.abs(Yf[r.row_of_slot[t, j]])
                n[t] += 1
    bound = np.maximum(n - 1, 0)[:, None] * 2.0 ** -24 * mass
    assert (np.abs(out - exact) <= bound).all()
    outbf = oracle.combine(idx, r.row_of_slot, Y, E, out="bf16")
    np.testing.assert_array_equal(outbf, torch_bf16(out.astype(np.float32)))


# --------------------------------------------------------------------------
# combine backward: cached dispatch, dw closed form, adjoint identity
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
def test_combine_bwd_is_cached_dispatch_and_dw_closed_form(seed):
    rng = np.random.default_rng(400 + seed)
    T, E, k, H = 40, 12, 4, 512
    EL, lb = (E, 0) if seed < 2 else (5, 4)
    idx = inputs.random_routing(T, E, k, rng, p_invalid=0.2, allow_dup=(seed % 2 == 1))
    x = inputs.bf16_normal((T, H), rng)
    g = inputs.bf16_normal((T, H), rng)
    r = oracle.route(idx, E, lb, EL, P=3, x=x)
    gr, dw = oracle.combine_bwd(idx, r.row_of_slot, r.row_token, g, E, lb, EL, F=r.rows)
    # grad rows = the dispatch of grad_out along the same layout
    rg = oracle.route(idx, E, lb, EL, P=3, x=g)
    np.testing.assert_array_equal(gr, rg.rows)
    # identity experts (F = dispatched x): dw[t,j] = <g_t, x_t> for local slots
    gd = f32_of_bf16(g).astype(np.float64)
    xd = f32_of_bf16(x).astype(np.float64)
    ref = np.einsum("th,th->t", gd, xd)
    mass = np.einsum("th,th->t", np.abs(gd), np.abs(xd))
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            if lb <= e < lb + EL:
                assert abs(dw[t, j] - ref[t]) <= 1e-6 * abs(ref[t]) + 1e-12 * mass[t]
            else:
                assert dw[t, j] == 0.0


def test_dw_exact_on_integer_inputs():
    rng = np.random.default_rng(9)
    T, E, k, H = 30, 6, 3, 256
    idx = inputs.random_routing(T, E, k, rng, p_invalid=0.2)
    g = torch_bf16(rng.integers(-8, 9, size=(T, H)).astype(np.float32))
    r = oracle.route(idx, E, P=2)
    F = torch_bf16(rng.integers(-8, 9, size=(r.R, H)).astype(np.float32))
    _, dw = oracle.combine_bwd(idx, r.row_of_slot, r.row_token, g, E, F=F)
    gi = f32_of_bf16(g).astype(np.int64)
    Fi = f32_of_bf16(F).astype(np.int64)
    for t in range(T):
        for j in range(k):
            if idx[t, j] >= 0:
                assert dw[t, j] == float(gi[t] @ Fi[r.row_of_slot[t, j]])


@pytest.mark.parametrize("seed", range(3))
def test_adjoint_identity(seed):
    # <combine(Y), G> == <Y, combine_bwd(G)> (exact with small-integer inputs)
    rng = np.random.default_rng(500 + seed)
    T, E, k, H = 48, 9, 3, 256
    idx = inputs.random_routing(T, E, k, rng, p_invalid=0.3, allow_dup=(seed == 2))
    r = oracle.route(idx, E, 2, 5, P=4, sync_free=True, C=oracle.capacity_min(T, k, 5, 4))
    Y = torch_bf16(rng.integers(-4, 5, size=(r.R, H)).astype(np.float32))
    G = torch_bf16(rng.integers(-4, 5, size=(T, H)).astype(np.float32))
    out = oracle.combine(idx, r.row_of_slot, Y, E, 2, 5, out="f32").astype(np.float64)
    gr, _ = oracle.combine_bwd(idx, r.row_of_slot, r.row_token, G, E, 2, 5)
    lhs = float((out * f32_of_bf16(G)).sum())
    rhs = float((f32_of_bf16(Y).astype(np.float64) * f32_of_bf16(gr)).sum())
    assert lhs == rhs


# --------------------------------------------------------------------------
# edge cases named by the review of _indices_to_multihot and the argument rules
# --------------------------------------------------------------------------

def test_edge_all_invalid():
    idx = -np.ones((5, 3), int)
    r = oracle.route(idx, 4, P=4, x=inputs.bf16_normal((5, 256), np.random.default_rng(0)))
    assert r.rc == oracle.OK and r.total == 0 and r.map.sum() == 0
    assert (r.row_of_slot == -1).all()
    out = oracle.combine(idx, r.row_of_slot, np.zeros((0, 256), np.uint16), 4)
    assert (out == 0).all()


def test_edge_duplicates_collapse():
    idx = np.array([[2, 2, 1], [0, 0, 0]])
    w = np.array([[0.25, 0.5, 0.125], [1.0, 2.0, 4.0]], np.float32)
    r = oracle.route(idx, 3, w=w, want_probs=True)
    assert r.flags & oracle.FLAG_DUP
    np.testing.assert_array_equal(r.tpe, [1, 1, 1])
    assert r.row_of_slot[0, 0] == r.row_of_slot[0, 1]
    assert len(set(r.row_of_slot[1])) == 1
    assert r.row_w[r.row_of_slot[0, 0]] == np.float32(0.75)
    assert r.row_w[r.row_of_slot[1, 0]] == np.float32(7.0)
    assert r.probs[0, 2] == np.float32(0.75) and r.probs[1, 0] == np.float32(7.0)


def test_edge_topk1_single_token_and_empty():
    r = oracle.route(np.array([[3]]), 5, P=8)
    np.testing.assert_array_equal(r.tpe, [0, 0, 0, 1, 0])
    assert r.total == 8 and r.row_of_slot[0, 0] == 0
    r0 = oracle.route(np.zeros((0, 4), int), 5, P=8)
    assert r0.rc == oracle.OK and r0.total == 0


def test_edge_out_of_range_ids_flagged_and_dropped():
    idx = np.array([[0, 7, -3], [1, -1, 2]])
    r = oracle.route(idx, 3)
    assert r.rc == oracle.ERR_INDEX and r.flags & oracle.FLAG_BAD_ID
    np.testing.assert_array_equal(r.map, expected_map(np.where((idx >= -1) & (idx < 3), idx, -1), 3))
    assert r.row_of_slot[0, 1] == -1 and r.row_of_slot[0, 2] == -1


def test_argument_rules():
    assert oracle.check_hidden(0) == oracle.ERR_HIDDEN
    assert oracle.check_hidden(384) == oracle.ERR_HIDDEN
    assert oracle.check_hidden(768) == oracle.OK
    assert oracle.check_args(10, 0, 8, 0, 8, 1) == oracle.ERR_ARG
    assert oracle.check_args(10, 2, 8, 4, 5, 1) == oracle.ERR_ARG
    assert oracle.check_args(10, 2, 8, 0, 8, 0) == oracle.ERR_ARG
    assert oracle.check_args(-1, 2, 8, 0, 8, 1) == oracle.ERR_ARG
    assert oracle.check_args(10, 2, 8, 0, 8, 2, True, 27) == oracle.ERR_CAPACITY
    assert oracle.check_args(10, 2, 8, 0, 8, 2, True, 28) == oracle.OK


# --------------------------------------------------------------------------
# the five workloads: generator + oracle invariants at full size (metadata)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_invariants(name):
    wl = inputs.WORKLOADS[name]
    case = inputs.make_case(wl, hidden=False)
    r = oracle.route(case.idx, wl.E, wl.lb, wl.num_local, wl.P, sync_free=wl.sync_free,
                     C=wl.cap if wl.sync_free else 0, w=case.w)
    assert r.rc == oracle.OK
    pairs = distinct_local_pairs(case.idx.astype(np.int64), wl.E, wl.lb, wl.num_local)
    assert r.tpe.sum() == len(pairs)
    np.testing.assert_array_equal(
        r.off, np.concatenate([[0], np.cumsum(-(-r.tpe // wl.P) * wl.P)]))
    if wl.sync_free:
        assert r.R == wl.cap and (r.row_expert[r.total:] == wl.num_local).all()
    # weights of every token's valid slots sum to ~1 (renormalised in fp32)
    if wl.invalid_slot_frac == 0:
        np.testing.assert_allclose(case.w.sum(1), 1.0, rtol=1e-5)
    if name == "h4096_rank_share":
        active = (r.map[:, :16].sum(1) > 0).mean()
        assert abs(active - 0.6674) < 0.02  # 1 - C(112,8)/C(128,8)
    if name == "skewed":
        assert r.tpe.max() > 20 * max(r.tpe.min(), 1)
        assert abs((case.idx == -1).all(1).mean() - 0.01) < 0.005


def test_dw_products_are_exact_beyond_fp32_range():
    # R12: each bf16 x bf16 product is taken exactly; 2^100 * 2^100 overflows
    # fp32 but the exact dot 2^200 - 2^200 + 1 = 1 is representable
    T, E, k, H = 1, 1, 1, 256
    idx = np.array([[0]])
    g = np.zeros((T, H), np.float32)
    F = np.zeros((1, H), np.float32)
    g[0, :3] = [2.0 ** 100, -(2.0 ** 100), 1.0]
    F[0, :3] = [2.0 ** 100, 2.0 ** 100, 1.0]
    r = oracle.route(idx, E)
    _, dw = oracle.combine_bwd(idx, r.row_of_slot, r.row_token, torch_bf16(g), E, F=torch_bf16(F))
    assert dw[0, 0] == 1.0


# --------------------------------------------------------------------------
# dispatch backward: the adjoint of dispatch (tokens and routing weights)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
def test_dispatch_bwd_is_the_adjoint_of_dispatch(seed):
    # <dispatch(x), G> == <x, dispatch_bwd(G)> and <row_w(w), g> == <w, grad_w(g)>,
    # exact on small-integer data (every sum is exact in fp32 and fp64)
    rng = np.random.default_rng(600 + seed)
    T, E, k, H = 40, 10, 4, 256
    EL, lb, P = (E, 0, 3) if seed % 2 == 0 else (6, 2, 2)
    sync_free = seed >= 2
    idx = inputs.random_routing(T, E, k, rng, p_invalid=0.25, allow_dup=(seed % 2 == 1))
    x = torch_bf16(rng.integers(-4, 5, size=(T, H)).astype(np.float32))
    w = rng.integers(-3, 4, size=(T, k)).astype(np.float32)
    C = oracle.capacity_min(T, k, EL, P) if sync_free else 0
    r = oracle.route(idx, E, lb, EL, P, sync_free=sync_free, C=C, w=w, x=x)
    G = torch_bf16(rng.integers(-4, 5, size=(r.R, H)).astype(np.float32))
    g = rng.integers(-3, 4, size=r.R).astype(np.float32)
    gx, gw = oracle.dispatch_bwd(idx, r.row_of_slot, G, E, lb, EL, grad_row_w=g, out="f32")
    lhs = float((f32_of_bf16(r.rows).astype(np.float64) * f32_of_bf16(G)).sum())
    rhs = float((f32_of_bf16(x).astype(np.float64) * gx).sum())
    assert lhs == rhs
    assert float((r.row_w.astype(np.float64) * g).sum()) == float((w.astype(np.float64) * gw).sum())
    # slots without a local row get no weight gradient
    no_row = r.row_of_slot < 0
    assert (gw[no_row] == 0).all()


def test_dispatch_bwd_inverts_top1_dispatch():
    rng = np.random.default_rng(8)
    T, E = 200, 12
    idx = rng.integers(0, E, size=(T, 1))
    x = inputs.bf16_normal((T, 512), rng)
    r = oracle.route(idx, E, P=4, x=x)
    gx, _ = oracle.dispatch_bwd(idx, r.row_of_slot, r.rows, E)
    np.testing.assert_array_equal(gx, x)
