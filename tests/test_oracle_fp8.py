"""Pins of the oracle's FP8 dispatch (readings R14..R17 of moe_oracle.c).

The element format is pinned to facts the OCP 8-bit floating point
specification fixes for E4M3 (largest finite 448, smallest normal 2^-6,
smallest subnormal 2^-9, one NaN pattern per sign) and, value by value, to an
independent implementation of the same rounding: torch's float8_e4m3fn cast on
the CPU.  The quantization is pinned by its invariants (each block's largest
magnitude lands on +-448, the error bound of a 3-bit mantissa, zero blocks),
by a hand-worked block, and the dispatch by its relation to the bf16 dispatch.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from combine_topk_idx_multihot_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fp8_block.json")


def torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def bf16_bits(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def test_format_facts():
    assert oracle.e4m3_value(0x7E) == 448.0            # largest finite
    assert oracle.e4m3_value(0x08) == 2.0 ** -6         # smallest normal
    assert oracle.e4m3_value(0x07) == 7 * 2.0 ** -9     # largest subnormal
    assert oracle.e4m3_value(0x01) == 2.0 ** -9         # smallest subnormal
    assert oracle.e4m3_value(0x38) == 1.0               # exponent field = bias
    assert oracle.e4m3_value(0xC0) == -2.0
    assert oracle.e4m3_value(0x80) == 0.0 and np.signbit(oracle.e4m3_value(0x80))
    assert np.isnan(oracle.e4m3_value(0x7F)) and np.isnan(oracle.e4m3_value(0xFF))
    finite = [oracle.e4m3_value(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(finite, finite[1:]))  # codes ordered by value


def test_every_code_rounds_to_itself():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    vals = np.array([oracle.e4m3_value(c) for c in codes], np.float32)
    np.testing.assert_array_equal(oracle.e4m3_round(vals), codes)


def _sweep():
    pos = np.array([oracle.e4m3_value(c) for c in range(0x7F)], np.float64)
    mids = (pos[:-1] + pos[1:]) / 2                   # exact in fp32: the ties
    m32 = mids.astype(np.float32)
    near = np.concatenate([np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9)),
                           m32])
    rng = np.random.default_rng(7)
    logu = np.float32(2.0) ** rng.uniform(-12, np.log2(448), 20000).astype(np.float32)
    lin = rng.uniform(0, 448, 20000).astype(np.float32)
    v = np.concatenate([pos.astype(np.float32), near, logu, lin, [0.0, 1e-30, 448.0]]).astype(
        np.float32)
    v = v[np.abs(v) <= 448]
    return np.concatenate([v, -v])


def test_rounding_matches_torch_float8_e4m3fn():
    v = _sweep()
    np.testing.assert_array_equal(oracle.e4m3_round(v), torch_e4m3(v))


def test_ties_go_to_the_even_code():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39); 1.1875 between
    # 1.125 (0x39) and 1.25 (0x3A); 2^-10 halfway between 0 and 2^-9;
    # 432 halfway between 416 (0x7D) and 448 (0x7E)
    got = oracle.e4m3_round([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 432.0, -1.0625])
    assert list(got) == [0x38, 0x3A, 0x00, 0x02, 0x7E, 0xB8]


def test_hand_worked_block():
    """A block whose largest magnitude is 448 has scale exactly 1, so its codes
    are the plain E4M3 roundings of its values (worked by hand in the fixture)."""
    g = json.load(open(GOLDEN))
    x = np.zeros((1, 128), np.float32)
    x[0, :len(g["x"])] = g["x"]
    q, s = oracle.fp8_quantize(bf16_bits(x))
    assert s[0, 0] == np.float32(1.0)
    assert [int(c) for c in q[0, :len(g["x"])]] == [int(c, 16) for c in g["codes"]]
    assert not q[0, len(g["x"]):].any()


def test_quantize_invariants():
    rng = np.random.default_rng(3)
    T, H = 64, 1024
    x = inputs.bf16_normal((T, H), rng)
    x[3] = 0                                              # an all-zero token
    x[5, :128] = bf16_bits(rng.normal(0, 1e-6, 128))       # a block below the floor
    x[7, 256:384] = bf16_bits(rng.normal(0, 100.0, 128))   # a large-valued block
    q, s = oracle.fp8_quantize(x)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    deq = np.vectorize(oracle.e4m3_value)(q).astype(np.float64)
    sb = np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(deq * sb - xf)
    # half a unit in the last place of a 3-bit mantissa (2^-4 relative), or
    # half the smallest subnormal step (2^-10 in code units) below 2^-6; plus
    # the roundings of the scale and of x * inv (a few fp32 ulps)
    bound = np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * sb) * (1 + 1e-6) + 1e-6 * np.abs(xf)
    assert np.all(err <= bound)
    blk = np.abs(xf).reshape(T, H // 128, 128).max(axis=2)
    big = blk >= 1e-4
    qmax = np.abs(deq).reshape(T, H // 128, 128).max(axis=2)
    assert np.all(qmax[big] == 448.0)                     # the block maximum lands on 448
    assert np.all(s[3] == np.float32(np.float32(1e-4) / np.float32(448.0)))
    assert not q[3].any()                                 # zero in, zero codes out
    assert s[5, 0] == s[3, 0]                             # the floor applies
    assert np.all(s[~big] == s[3, 0])
    assert s[7, 2] > 0.1


def test_dispatch_fp8_follows_the_bf16_dispatch():
    rng = np.random.default_rng(9)
    T, k, E, H, P = 200, 4, 16, 512, 8
    idx = inputs.random_routing(T, E, k, rng, p_invalid=0.1, allow_dup=True)
    x = inputs.bf16_normal((T, H), rng)
    for sync_free in (False, True):
        C = oracle.capacity_min(T, k, 12, P) if sync_free else 0
        ref = oracle.route(idx, E, 2, 12, P, sync_free=sync_free, C=C, x=x)
        q, s = oracle.dispatch_fp8(x, ref.row_token)
        data = ref.row_token >= 0
        q2, s2 = oracle.fp8_quantize(ref.rows[data])       # quantize the bf16 rows instead
        np.testing.assert_array_equal(q[data], q2)
        np.testing.assert_array_equal(s[data], s2)
        assert not q[~data].any() and not s[~data].any()   # pad and sentinel rows
        assert q.shape == (ref.R, H) and s.shape == (ref.R, H // 128)


def test_dispatch_fp8_rejects_bad_hidden():
    with pytest.raises(ValueError):
        oracle.dispatch_fp8(np.zeros((2, 200), np.uint16), np.zeros(1, np.int32))
