"""PreparedDispatch, PreparedCombine and PreparedCombineBwd on the GPU.

The binding's prepared calls over reused, worst-case sized buffers give exactly
what the plain calls give for each step's R (rows [0, R) of the dispatch, the
combine's output, the grad rows and dw), for successive routings through the
same handle; R past the buffers' capacity is refused before any launch, and
R = 0 launches nothing.
"""
import numpy as np
import pytest
import torch

from combine_topk_idx_multihot_amd import binding as B
from combine_topk_idx_multihot_amd import inputs
from test_gpu_parity import gpu, say  # noqa: F401 (gpu: fixture)

pytestmark = pytest.mark.gpu


def test_prepared_dispatch_matches_fresh_buffers():
    T, H, E, k, P = 1500, 768, 48, 6, 8
    say(f"[prepared] eager T={T} H={H} E={E} k={k} P={P}")
    d = B.make_desc(T, k, E, 0, E, P, B.MOE_EAGER, False, 0)
    cap = B.moe_capacity_min(d)
    h = B.alloc_handle(d)
    x = torch.randn((T, H), device="cuda").to(torch.bfloat16)
    w = torch.rand((T, k), device="cuda")
    rows = torch.full((cap, H), 7.0, dtype=torch.bfloat16, device="cuda")
    row_w = torch.empty(cap, dtype=torch.float32, device="cuda")
    rt = torch.empty(cap, dtype=torch.int32, device="cuda")
    re = torch.empty(cap, dtype=torch.int32, device="cuda")
    prep = B.PreparedDispatch(d, h, x, H, rows, w, row_w, rt, re)
    assert prep.capacity == cap
    for seed in (1, 2, 3):
        rng = np.random.default_rng(seed)
        idx = inputs.random_routing(T, E, k, rng, p_invalid=0.1 * seed)
        B.moe_route_build(d, torch.from_numpy(idx.astype(np.int32)).cuda(), h)
        R = h.total
        prep(R)
        ref = B.dispatch(d, h, x, w)
        torch.cuda.synchronize()
        say(f"  seed {seed}: R={R} of {cap}")
        assert torch.equal(rows[:R], ref[0])
        assert torch.equal(row_w[:R], ref[1])
        assert torch.equal(rt[:R], ref[2])
        assert torch.equal(re[:R], ref[3])
    with pytest.raises(B.MoeError):
        prep(cap + 1)
    with pytest.raises(B.MoeError):
        prep(-1)
    prep(0)
    torch.cuda.synchronize()


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_prepared_combine_and_backward_match_plain_calls(out_dtype):
    """PreparedCombine and PreparedCombineBwd over worst-case buffers give
    exactly what moe_combine and moe_combine_bwd give for each step's R,
    including dw; R past the buffers is refused."""
    T, H, E, k, P = 1200, 512, 40, 6, 4
    say(f"[prepared] combine + backward T={T} H={H} E={E} k={k} P={P} out={out_dtype}")
    d = B.make_desc(T, k, E, 0, E, P, B.MOE_EAGER, False, 0)
    cap = B.moe_capacity_min(d)
    h = B.alloc_handle(d)
    Y = torch.randn((cap, H), device="cuda").to(torch.bfloat16)
    F = torch.randn((cap, H), device="cuda").to(torch.bfloat16)
    g = torch.randn((T, H), device="cuda").to(torch.bfloat16)
    out = torch.empty((T, H), dtype=out_dtype, device="cuda")
    gr = torch.full((cap, H), 3.0, dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    comb = B.PreparedCombine(d, h, Y, H, out)
    bwd = B.PreparedCombineBwd(d, h, g, H, gr, F, dw)
    assert comb.capacity == cap and bwd.capacity == cap
    for seed in (4, 5):
        rng = np.random.default_rng(seed)
        idx = inputs.random_routing(T, E, k, rng, p_invalid=0.2)
        B.moe_route_build(d, torch.from_numpy(idx.astype(np.int32)).cuda(), h)
        R = h.total
        comb(R)
        bwd(R)
        ref_out = torch.empty_like(out)
        B.moe_combine(d, h, Y[:R], H, R, ref_out)
        ref_gr = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
        ref_dw = torch.empty_like(dw)
        B.moe_combine_bwd(d, h, g, H, R, ref_gr, F[:R], ref_dw)
        torch.cuda.synchronize()
        say(f"  seed {seed}: R={R} of {cap}")
        assert torch.equal(out.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                           ref_out.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32))
        assert torch.equal(gr[:R].view(torch.int16), ref_gr.view(torch.int16))
        assert torch.equal(dw.view(torch.int32), ref_dw.view(torch.int32))
    for call in (comb, bwd):
        with pytest.raises(B.MoeError):
            call(cap + 1)
        with pytest.raises(B.MoeError):
            call(-1)
