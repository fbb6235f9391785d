"""Row arrays past 4 GiB on the GPU.

A sync-free layer with T = 40000, k = 8, E = 64 (all local), P = 4 and H = 8192
has a capacity of 320192 rows of 16 KiB: each row array is 5.2 GB, and row
262144 starts exactly at byte 2^32.  The routing metadata is compared whole
with the oracle.  The rows and grad rows are compared on samples: rows around
the 4 GiB boundary, around the routed total, the last rows, random rows, and
the rows of sampled tokens.  For the sampled tokens, the oracle computes the
combine and the combine backward (grad rows and dw) on the compact
sub-problem they make up.  The zero tail is checked whole on the device.  The
FP8 dispatch of the same layer is checked the same way; its E4M3 rows are H
bytes, so the same boundary row starts at byte 2^31 of the code array.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_topk_idx_multihot_amd import binding as B
from combine_topk_idx_multihot_amd import inputs
from test_gpu_parity import check_dw, gpu, say, to_np_u16  # noqa: F401 (gpu: fixture)

pytestmark = pytest.mark.gpu

T, E, k, P, H = 40000, 64, 8, 4, 8192
BOUNDARY_ROW = (1 << 32) // (2 * H)  # first row at or past byte 2^32


def rows_np(t, idx):
    """Rows `idx` of a device bf16 [R,H] tensor, as uint16 bits on the host."""
    return to_np_u16(t.index_select(0, torch.from_numpy(idx.astype(np.int64)).cuda()))


def test_rows_past_4gib():
    rng = np.random.default_rng(4242)
    idx = inputs.random_routing(T, E, k, rng, p_invalid=0.05)
    w = rng.random((T, k), dtype=np.float32)
    C = oracle.capacity_min(T, k, E, P)
    assert C * H * 2 > (1 << 32) + (1 << 29), C  # well past 4 GiB
    say(f"[large] sync-free T={T} k={k} E={E} P={P} H={H} C={C}: "
        f"{C * H * 2 / 1e9:.2f} GB per row array")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    x = torch.randn((T, H), generator=gen, device="cuda").to(torch.bfloat16)
    g = torch.randn((T, H), generator=gen, device="cuda").to(torch.bfloat16)
    F = torch.randn((C, H), generator=gen, device="cuda").to(torch.bfloat16)
    d = B.make_desc(T, k, E, 0, E, P, B.MOE_SYNC_FREE, False, C)
    h = B.alloc_handle(d)
    w_t = torch.from_numpy(w).cuda()
    B.moe_route_build(d, torch.from_numpy(idx.astype(np.int32)).cuda(), h)
    rows, row_w, rt, re = B.dispatch(d, h, x, w_t)
    out = B.combine(d, h, rows)
    grad_rows, dw = B.combine_bwd(d, h, g, C, F)
    torch.cuda.synchronize()

    # metadata, whole
    ref = oracle.route(idx, E, 0, E, P, sync_free=True, C=C, w=w)
    assert ref.rc == oracle.OK
    np.testing.assert_array_equal(h.row_of_slot.cpu().numpy(), ref.row_of_slot)
    np.testing.assert_array_equal(h.padded_offsets.cpu().numpy(), ref.off)
    np.testing.assert_array_equal(h.tokens_per_expert.cpu().numpy(), ref.tpe)
    np.testing.assert_array_equal(rt.cpu().numpy(), ref.row_token)
    np.testing.assert_array_equal(re.cpu().numpy(), ref.row_expert)
    np.testing.assert_array_equal(row_w.cpu().numpy().view(np.uint32), ref.row_w.view(np.uint32))
    total = int(ref.total)
    assert BOUNDARY_ROW < total < C

    # sampled tokens and the rows they use
    S = np.unique(np.concatenate([rng.choice(T, 300, replace=False), [0, T - 1]]))
    ros_S = ref.row_of_slot[S]
    U = np.unique(ros_S[ros_S >= 0])
    assert (U >= BOUNDARY_ROW).any() and (U < BOUNDARY_ROW).any()

    # rows: data rows are x's token rows, the others zero, bit for bit
    sample = np.unique(np.concatenate([
        np.arange(BOUNDARY_ROW - 4, BOUNDARY_ROW + 4), np.arange(total - 4, total + 4),
        np.arange(C - 4, C), rng.choice(C, 2000, replace=False), U]))
    tok = ref.row_token[sample]
    want_x = rows_np(x, np.maximum(tok, 0))
    want_x[tok < 0] = 0
    np.testing.assert_array_equal(rows_np(rows, sample), want_x)
    want_g = rows_np(g, np.maximum(tok, 0))
    want_g[tok < 0] = 0
    np.testing.assert_array_equal(rows_np(grad_rows, sample), want_g)
    # the zero tail, whole (a device-side reduction over 0.26 GB per array)
    assert not bool((rows[total:].view(torch.int16) != 0).any())
    assert not bool((grad_rows[total:].view(torch.int16) != 0).any())

    # combine and the combine backward of the sampled tokens, from the oracle
    # on the compact sub-problem (rows U renumbered 0..|U|-1)
    pos = {int(r): i for i, r in enumerate(U)}
    ros_c = np.where(ros_S >= 0, np.vectorize(lambda r: pos.get(int(r), -1))(ros_S), -1)
    ros_c = ros_c.astype(np.int32)
    tok_of_S = {int(t): i for i, t in enumerate(S)}
    rt_c = np.array([tok_of_S[int(ref.row_token[r])] for r in U], np.int32)
    Y_c = rows_np(rows, U)
    g_S = rows_np(g, S)
    F_c = rows_np(F, U)
    out_exp = oracle.combine(idx[S], ros_c, Y_c, E)
    np.testing.assert_array_equal(rows_np(out, S), out_exp)
    gr_c, dw_c = oracle.combine_bwd(idx[S], ros_c, rt_c, g_S, E, F=F_c, R=len(U))
    np.testing.assert_array_equal(rows_np(grad_rows, U), gr_c)
    check_dw(dw.cpu().numpy()[S], dw_c, idx[S], ros_c, g_S, F_c, 0, E, E)
    say(f"  total={total}, {len(sample)} rows and {len(S)} tokens sampled, "
        f"{int((U >= BOUNDARY_ROW).sum())} of their rows past 4 GiB")

    # the FP8 dispatch of the same layer: E4M3 rows of H bytes, so the same
    # boundary row starts at byte 2^31 of the code array
    del grad_rows, F
    q, sc, rw8, rt8, re8 = B.dispatch_fp8(d, h, x, w_t)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(rt8.cpu().numpy(), ref.row_token)
    np.testing.assert_array_equal(re8.cpu().numpy(), ref.row_expert)
    np.testing.assert_array_equal(rw8.cpu().numpy().view(np.uint32), ref.row_w.view(np.uint32))
    sel = torch.from_numpy(sample.astype(np.int64)).cuda()
    q_s = q.view(torch.uint8).index_select(0, sel).cpu().numpy()
    sc_s = sc.index_select(0, sel).cpu().numpy()
    data = tok >= 0
    toks = np.unique(tok[data])
    compact = np.searchsorted(toks, tok[data]).astype(np.int32)
    q_exp, s_exp = oracle.dispatch_fp8(rows_np(x, toks), compact)
    np.testing.assert_array_equal(q_s[data], q_exp)
    np.testing.assert_array_equal(sc_s[data].view(np.uint32), s_exp.view(np.uint32))
    assert not q_s[~data].any() and not sc_s[~data].any()
    assert not bool((q.view(torch.uint8)[total:] != 0).any())
    assert not bool((sc[total:] != 0).any())
