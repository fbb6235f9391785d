"""GPU parity on seeded random configurations: token counts, slot counts,
expert ranges, pad multiples, hidden sizes, both modes, both id widths,
empty slots, repeated ids and out-of-range ids, drawn from one master seed.

Every call of the path runs on each configuration (route, dispatch, combine,
combine backward with dw, dispatch backward, FP8 dispatch) and is compared
with the oracle exactly as in test_gpu_parity / test_gpu_fp8.
"""
import numpy as np
import pytest

import oracle
from combine_topk_idx_multihot_amd import inputs
from test_gpu_fp8 import RunFp8, check_all_rows, check_meta, check_sampled_rows
from test_gpu_parity import Run, check_against_oracle, gpu, say  # noqa: F401 (gpu: fixture)

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
