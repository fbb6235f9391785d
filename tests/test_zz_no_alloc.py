"""moe_route_build_noalloc on the GPU: the route with its scratch in the
library's fixed per-GPU array, for callers that cannot allocate.

Held bit for bit against moe_route_build with a workspace of its own on the
same inputs: multihot map, multihot probs, tokens_per_expert, padded offsets,
row of every slot, device status and host status.  Several calls in a row
share the one array, each smaller than the one before (the three-launch route
of a count table past 64 Ki entries, the two-launch route, a one-workgroup
route), so every call finds the previous call's leftovers there; eager and
sync-free.  A dispatch along the handle it built must equal the dispatch
along moe_route_build's handle.  Routes too large for the array, and handles
that bring a workspace, are refused before anything is launched.
"""
import numpy as np
import pytest
import torch

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


# (T, E, k, lb, EL, P): largest first
SIZES = [
    (33000, 128, 8, 0, 128, 16),  # 516 route blocks x 128 local: three launches
    (4096, 128, 8, 0, 128, 16),   # 64 blocks: count pass + finishing pass
    (60, 64, 8, 8, 32, 4),        # one counting workgroup
]


def route_both(d, idx_t, w_t):
    """The same route through moe_route_build (own workspace) and
    moe_route_build_noalloc (the library's array); returns both handles and
    probs, host status included."""
    T, E = d.T, d.E
    h_ref = B.alloc_handle(d)
    p_ref = torch.empty((T, E), dtype=torch.float32, device="cuda")
    B.moe_route_build(d, idx_t, h_ref, w_t, p_ref)
    h_na = B.alloc_handle(d, with_workspace=False)
    # outputs poisoned, so that a word the call fails to write shows up
    h_na.row_of_slot.fill_(-77)
    h_na.tokens_per_expert.fill_(-77)
    h_na.padded_offsets.fill_(-77)
    h_na.routing_map.fill_(0xA5)
    p_na = torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda")
    B.moe_route_build_noalloc(d, idx_t, h_na, w_t, p_na)
    torch.cuda.synchronize()
    return (h_ref, p_ref), (h_na, p_na)


def assert_same_route(ref, got, eager):
    (h_ref, p_ref), (h_na, p_na) = ref, got
    for name in ("routing_map", "tokens_per_expert", "padded_offsets", "row_of_slot", "status"):
        assert torch.equal(getattr(h_ref, name), getattr(h_na, name)), name
    assert torch.equal(p_ref.view(torch.int32), p_na.view(torch.int32))
    if eager:
        np.testing.assert_array_equal(h_ref.host_status.numpy()[:3], h_na.host_status.numpy()[:3])


@pytest.mark.parametrize("sync_free", [False, True], ids=["eager", "sync_free"])
def test_noalloc_route_equals_route_build_on_calls_in_a_row(sync_free):
    last = None
    for i, (T, E, k, lb, EL, P) in enumerate(SIZES):
        rng = np.random.default_rng([91, i, int(sync_free)])
        idx = inputs.random_routing(T, E, k, rng, p_invalid=0.03)
        w = rng.random((T, k), dtype=np.float32)
        C = B.moe_capacity_min(B.make_desc(T, k, E, lb, EL, P)) if sync_free else 0
        d = B.make_desc(T, k, E, lb, EL, P, B.MOE_SYNC_FREE if sync_free else B.MOE_EAGER,
                        False, C)
        # the route's full workspace (scratch plus the row list, which this
        # call does not write) bounds what it needs of the fixed array
        ws = B.moe_route_workspace_size(d)
        assert ws <= B.MOE_NOALLOC_SCRATCH_BYTES
        if last is not None:
            assert T < last  # each call's input smaller than the one before
        last = T
        say(f"[noalloc] call {i}: T={T} E={E} k={k} lb={lb} EL={EL} P={P} "
            f"sync_free={sync_free} scratch={ws} B")
        idx_t = torch.from_numpy(idx.astype(np.int32)).cuda()
        w_t = torch.from_numpy(w).cuda()
        ref, got = route_both(d, idx_t, w_t)
        assert_same_route(ref, got, not sync_free)
        # a dispatch along each handle: the same rows and metadata
        H = 256
        x = torch.randn((T, H), device="cuda").to(torch.bfloat16)
        a = B.dispatch(d, ref[0], x, w_t)
        b = B.dispatch(d, got[0], x, w_t)
        torch.cuda.synchronize()
        for ta, tb, name in zip(a, b, ("rows", "row_w", "row_token", "row_expert")):
            assert torch.equal(ta.view(torch.int16) if ta.dtype == torch.bfloat16 else ta,
                               tb.view(torch.int16) if tb.dtype == torch.bfloat16 else tb), name


def test_noalloc_route_repeated_on_one_stream():
    """Two different routings of one shape queued back to back on one stream:
    the second finds the first's scratch and must still equal its own
    moe_route_build."""
    T, E, k, P = 5000, 96, 6, 8
    d = B.make_desc(T, k, E, 0, E, P, B.MOE_SYNC_FREE, False,
                    B.moe_capacity_min(B.make_desc(T, k, E, 0, E, P)))
    s = torch.cuda.Stream()
    hs, refs = [], []
    for rep in range(2):
        rng = np.random.default_rng([92, rep])
        idx_t = torch.from_numpy(inputs.random_routing(T, E, k, rng, p_invalid=0.1)
                                 .astype(np.int32)).cuda()
        h_ref = B.alloc_handle(d)
        B.moe_route_build(d, idx_t, h_ref)
        refs.append(h_ref)
        h = B.alloc_handle(d, with_workspace=False)
        hs.append((h, idx_t))
    torch.cuda.synchronize()
    say("[noalloc] two routes queued on one stream")
    with torch.cuda.stream(s):
        for h, idx_t in hs:
            B.moe_route_build_noalloc(d, idx_t, h, stream=s)
    torch.cuda.synchronize()
    for (h, _), h_ref in zip(hs, refs):
        for name in ("routing_map", "tokens_per_expert", "padded_offsets", "row_of_slot", "status"):
            assert torch.equal(getattr(h_ref, name), getattr(h, name)), name


def test_noalloc_route_refuses_oversized_and_workspace():
    # 40000 tokens at k = 8 with 1024 local experts: 1250 route blocks x 1024
    # counts = 5 MB of scratch, past the 4 MiB array
    d = B.make_desc(40000, 8, 1024, 0, 1024, 1)
    assert B.moe_route_workspace_size(d) > B.MOE_NOALLOC_SCRATCH_BYTES
    h = B.alloc_handle(d, with_map=False, with_workspace=False)
    idx_t = torch.zeros((40000, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(B.MoeError) as e:
        B.moe_route_build_noalloc(d, idx_t, h)
    assert e.value.code == B.MOE_ERR_WORKSPACE
    assert "fixed" in B.last_error()
    d2 = B.make_desc(100, 2, 8)
    h2 = B.alloc_handle(d2)  # brings a workspace
    with pytest.raises(B.MoeError) as e:
        B.moe_route_build_noalloc(d2, torch.zeros((100, 2), dtype=torch.int32, device="cuda"), h2)
    assert e.value.code == B.MOE_ERR_ARG
