"""The reference kernels of libmoe_ceiling on the GPU write exactly what
include/moe_ceiling.h says: the fill zeroes the whole buffer, the copy
reproduces its source, the scatter zeroes exactly the rows a real
handle's row_of_slot names (every other row keeps its contents), and the
gather stores each token's fp32 sum of its named rows in slot order,
truncated to bf16 (or, read only, stores nothing), for ragged sizes and
every piece / segment size."""
import numpy as np
import pytest
import torch

from combine_topk_idx_multihot_amd import binding as B
from combine_topk_idx_multihot_amd import ceiling as C
from combine_topk_idx_multihot_amd import inputs
from test_gpu_parity import gpu, say  # noqa: F401 (gpu: fixture)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("pk", [1, 2, 4])
@pytest.mark.parametrize("nbytes", [16, 1024 * 63 + 16 * 7, 3 << 20])
def test_fill_and_copy(pk, nbytes):
    say(f"[ceiling] fill/copy {nbytes} B, {pk} KiB pieces")
    src = torch.randint(0, 255, (nbytes + 4096,), dtype=torch.uint8, device="cuda")
    dst = torch.full((nbytes + 4096,), 7, dtype=torch.uint8, device="cuda")
    C.copy(src[:nbytes], dst[:nbytes], piece_kib=pk)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert (dst[nbytes:] == 7).all()  # nothing past the end
    C.fill(dst[:nbytes], piece_kib=pk)
    torch.cuda.synchronize()
    assert (dst[:nbytes] == 0).all() and (dst[nbytes:] == 7).all()


@pytest.mark.parametrize("seg", [1, 2, 4])
def test_scatter_zeroes_exactly_the_named_rows(seg):
    rng = np.random.default_rng([5, seg])
    T, E, k, H, P = 777, 40, 6, 1280, 4
    idx = inputs.random_routing(T, E, k, rng, p_invalid=0.1, allow_dup=True)
    d = B.make_desc(T, k, E, 0, E, P)
    h, _ = B.route(d, torch.from_numpy(idx.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    R = h.total
    say(f"[ceiling] scatter T={T} k={k} R={R} H={H} seg={seg} KiB")
    rows = torch.full((R + 3, H), 1.5, dtype=torch.bfloat16, device="cuda")
    C.scatter(h.row_of_slot, rows[:R], seg_kib=seg)
    torch.cuda.synchronize()
    named = np.zeros(R + 3, bool)
    ros = h.row_of_slot.cpu().numpy()
    named[ros[ros >= 0]] = True
    got = rows.float().cpu().numpy()
    assert (got[named] == 0).all()
    assert (got[~named] == 1.5).all()


@pytest.mark.parametrize("seg", [1, 2, 4])
@pytest.mark.parametrize("H", [768, 2048])
def test_gather_sums_the_named_rows(seg, H):
    rng = np.random.default_rng([6, seg, H])
    T, E, k, P = 555, 40, 6, 4
    idx = inputs.random_routing(T, E, k, rng, p_invalid=0.1, allow_dup=True)
    d = B.make_desc(T, k, E, 0, E, P)
    h, _ = B.route(d, torch.from_numpy(idx.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    R = h.total
    say(f"[ceiling] gather T={T} k={k} R={R} H={H} seg={seg} KiB")
    Y_np = inputs.bf16_normal((R, H), rng)
    Y = torch.from_numpy(Y_np.view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.full((T + 2, H), 3.0, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    C.gather(h.row_of_slot, Y, None, sink, seg_kib=seg)  # read only: stores nothing
    torch.cuda.synchronize()
    assert int(sink[0]) == 0 and (out.float() == 3.0).all()
    C.gather(h.row_of_slot, Y, out[:T], seg_kib=seg)
    torch.cuda.synchronize()
    ros = h.row_of_slot.cpu().numpy()
    Yf = (Y_np.astype(np.uint32) << 16).view(np.float32)
    acc = np.zeros((T, H), np.float32)
    for j in range(k):  # slot order, a named row or +0
        r = ros[:, j]
        acc = acc + np.where((r >= 0)[:, None], Yf[np.maximum(r, 0)], np.float32(0))
    want = (acc.view(np.uint32) >> 16).astype(np.uint16)
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got[:T], want)
    assert (out[T:].float() == 3.0).all()


def test_workgroups_run_on_xcd_j_mod_8():
    """The combine backward numbers its workgroups so that the copy and dot
    workgroups of one token period land on one XCD, assuming workgroup j runs
    on XCD j mod 8 (MI355X in its one-partition mode).  Checked on this GPU
    from each workgroup's XCC_ID register."""
    m = C.xcd_map(8192).cpu().numpy()
    say(f"[xcd] XCDs seen: {sorted(set(m.tolist()))}")
    assert set(m.tolist()) == set(range(8))
    np.testing.assert_array_equal(m, np.arange(8192) % 8)
