"""PreparedDispatch on the GPU: the binding's dispatch over reused, worst-case
sized buffers gives, in rows [0, R), exactly what moe_dispatch gives in fresh
buffers of R rows, for successive routings through the same handle; R past the
buffers' capacity is refused before any launch, and R = 0 launches nothing.
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
