"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments with the documented codes before touching the GPU.

No kernel is launched here: every call below fails host validation, which runs
before any HIP call.
"""
import ctypes
import os
import re

import pytest

import oracle
from combine_topk_idx_multihot_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "moe_mi355x.h")
FAKE = 0x100000  # a 16-byte aligned non-NULL address; never dereferenced by validation


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))


def test_library_loads_and_exports_every_declared_symbol():
    L = B.lib()
    names = declared_functions()
    assert set(names) == set(B.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_desc_struct_layout_matches_header():
    assert ctypes.sizeof(B.Desc) == 48
    assert B.Desc.capacity.offset == 40
    assert ctypes.sizeof(B._Handle) == 7 * 8


def _desc(**kw):
    base = dict(T=100, k=8, E=128, local_begin=0, num_local=128, pad_multiple=16,
                mode=B.MOE_EAGER, idx_is_i64=False, capacity=0)
    base.update(kw)
    return B.make_desc(**base)


def _handle(ws_bytes=1 << 30):
    h = B._Handle(routing_map=FAKE, tokens_per_expert=FAKE, padded_offsets=FAKE,
                  row_of_slot=FAKE, status=FAKE, workspace=FAKE, workspace_bytes=ws_bytes)
    return h


def route_rc(d, ws_bytes=1 << 30, idx=FAKE, w=None, probs=None, host=FAKE, handle=None):
    h = handle if handle is not None else _handle(ws_bytes)
    return B.lib().moe_route_build(ctypes.byref(d), idx, w, probs, ctypes.byref(h), host, None)


def dispatch_rc(d, H=2048, R=10, x=FAKE, rows=FAKE, w=None, row_w=None):
    h = _handle()
    return B.lib().moe_dispatch(ctypes.byref(d), ctypes.byref(h), x, H, w, R, rows, row_w, None,
                                None, None)


def combine_rc(d, H=2048, R=10, Y=FAKE, out=FAKE, f32=0):
    h = _handle()
    return B.lib().moe_combine(ctypes.byref(d), ctypes.byref(h), Y, H, R, out, f32, None)


def bwd_rc(d, H=2048, R=10, g=FAKE, F=None, gr=FAKE, dw=None):
    h = _handle()
    return B.lib().moe_combine_bwd(ctypes.byref(d), ctypes.byref(h), g, F, H, R, gr, dw, None)


@pytest.mark.parametrize("H", [0, -256, 100, 384, 2049])
def test_hidden_must_be_multiple_of_256(H):
    d = _desc()
    for rc in (dispatch_rc(d, H=H), combine_rc(d, H=H), bwd_rc(d, H=H)):
        assert rc == B.MOE_ERR_HIDDEN
    assert "256" in B.last_error()


@pytest.mark.parametrize("field,value", [
    ("T", -1), ("k", 0), ("k", 65), ("E", 0), ("pad_multiple", 0), ("local_begin", -1),
    ("num_local", 0), ("num_local", 129), ("mode", 2), ("num_local", 1025),
])
def test_bad_desc_is_rejected(field, value):
    kw = {field: value}
    if field == "num_local" and value == 1025:
        kw["E"] = 2048
    d = _desc(**kw)
    assert route_rc(d) == B.MOE_ERR_ARG
    assert dispatch_rc(d) == B.MOE_ERR_ARG
    assert B.last_error()


def test_local_range_must_fit():
    assert route_rc(_desc(local_begin=120, num_local=16)) == B.MOE_ERR_ARG


def test_sync_free_capacity_rule():
    T, k, EL, P = 100, 8, 16, 4
    cmin = T * min(k, EL) + EL * (P - 1)
    d = _desc(T=T, k=k, num_local=EL, pad_multiple=P, mode=B.MOE_SYNC_FREE, capacity=cmin - 1)
    assert B.moe_capacity_min(d) == cmin == oracle.capacity_min(T, k, EL, P)
    assert route_rc(d) == B.MOE_ERR_CAPACITY
    assert "worst case" in B.last_error()
    d.capacity = cmin
    # sync-free rows must equal the capacity
    assert dispatch_rc(d, R=cmin - 1) == B.MOE_ERR_ARG


def test_capacity_min_matches_oracle_on_a_grid():
    for T in (0, 1, 7, 4096):
        for k in (1, 2, 8):
            for EL in (1, 4, 16, 128):
                for P in (1, 2, 16, 128):
                    d = _desc(T=T, k=k, num_local=EL, pad_multiple=P)
                    assert B.moe_capacity_min(d) == oracle.capacity_min(T, k, EL, P)


def test_workspace_rules():
    d = _desc()
    need = B.moe_route_workspace_size(d)
    assert need > 0
    assert route_rc(d, ws_bytes=need - 1) == B.MOE_ERR_WORKSPACE
    # only route_build needs the workspace (dispatch reads the route's row list
    # from it when it is there and walks tokens without it): dispatch gets past
    # the handle check with none and stops at a later rule (weights with no
    # row_w), launching nothing
    h = _handle(need - 1)
    h.workspace = None
    assert B.lib().moe_dispatch(ctypes.byref(d), ctypes.byref(h), FAKE, 2048, FAKE, 10, FAKE, None,
                                None, None, None) == B.MOE_ERR_ARG
    assert "row_w" in B.last_error()
    h = _handle()
    h.workspace = None
    assert route_rc(d, handle=h) == B.MOE_ERR_WORKSPACE
    assert B.lib().moe_route_workspace_size(ctypes.byref(_desc(k=0))) == 0


def route_blocks(T, k, EL):
    """The library's count of route blocks: blocks of 512 slots up to 512
    local experts (else 256), or one block of up to 2048 slots when its
    local experts are few (T <= 1024 // k with EL <= 256, or T <= 2048 // k
    with EL <= 64)."""
    if T == 0:
        return 0
    nblk = -(-T // ((512 if EL <= 512 else 256) // k))
    if nblk > 1 and (T <= 1024 // k and EL <= 256 or T <= 2048 // k and EL <= 64):
        return 1
    return nblk


def _up256(n):
    return (n + 255) // 256 * 256


@pytest.mark.parametrize("T,E,k,EL", [
    (4096, 128, 8, 128), (16384, 64, 8, 64), (1027, 16, 4, 16), (300, 8, 2, 8),
    (64, 128, 8, 128), (65, 128, 8, 128), (4096, 128, 8, 16), (4096, 128, 8, 32),
    (32768, 128, 8, 128), (32769, 128, 8, 128), (2100, 1024, 8, 1024), (1500, 8, 8, 2),
    (999, 32, 6, 32), (40000, 64, 8, 64), (700, 64, 1, 64), (0, 8, 2, 8)])
def test_workspace_size_follows_the_row_list_rule(T, E, k, EL):
    """moe_route_workspace_size: the route's scratch (per-block counts and
    flags), plus the row list exactly when the route spans several blocks,
    the count table stays within 65536 entries and k * EL >= 2 * E; the list
    is at least 8 bytes per (token, min(k, EL)) and at most that plus whole
    tiles of 512 tokens on each of the 8 XCDs."""
    d = _desc(T=T, E=E, k=k, num_local=EL, pad_multiple=1)
    nblk = route_blocks(T, k, EL)
    scratch = _up256(nblk * EL * 4) + _up256(nblk * 4)
    got = B.moe_route_workspace_size(d)
    listed = nblk > 1 and nblk * EL <= 65536 and k * EL >= 2 * E
    if not listed:
        assert got == max(scratch, 256)
        return
    kk = min(k, EL)
    extra = got - scratch
    assert 8 * T * kk <= extra <= _up256(8 * kk * (T + 8 * 512) + 8 * 8 * 3), (got, scratch)


def test_noalloc_route_rules():
    """moe_route_build_noalloc: a handle that brings a workspace, a route too
    large for the fixed array, and the route's own rules are all refused
    before any HIP call."""
    L = B.lib()

    def rc(d, h, w=None, probs=None, host=FAKE, idx=FAKE):
        return L.moe_route_build_noalloc(ctypes.byref(d), idx, w, probs, ctypes.byref(h), host,
                                         None)

    d = _desc()
    assert rc(d, _handle()) == B.MOE_ERR_ARG                      # a workspace it would ignore
    assert "workspace" in B.last_error()
    h = _handle(0)
    h.workspace = None
    h.workspace_bytes = 64
    assert rc(d, h) == B.MOE_ERR_ARG
    h.workspace_bytes = 0
    big = _desc(T=40000, E=1024, num_local=1024, pad_multiple=1)  # 1250 blocks x 1024 counts
    assert B.moe_route_workspace_size(big) > B.MOE_NOALLOC_SCRATCH_BYTES
    assert rc(big, h) == B.MOE_ERR_WORKSPACE
    assert "fixed" in B.last_error()
    assert rc(d, h, w=FAKE) == B.MOE_ERR_ARG                      # weights with nothing to write
    assert rc(d, h, probs=FAKE) == B.MOE_ERR_ARG                  # probs without weights
    assert rc(d, h, host=None) == B.MOE_ERR_ARG                   # eager needs the host status
    assert rc(d, h, idx=None) == B.MOE_ERR_ARG
    assert rc(_desc(k=0), h) == B.MOE_ERR_ARG
    assert rc(_desc(mode=B.MOE_SYNC_FREE, capacity=5), h) == B.MOE_ERR_CAPACITY


def test_noalloc_scratch_size_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES (\d+)u", src)
    assert m and int(m.group(1)) == B.MOE_NOALLOC_SCRATCH_BYTES == 4 << 20


def test_route_flag_pairs_are_never_ignored():
    d = _desc()
    assert route_rc(d, w=FAKE, probs=None) == B.MOE_ERR_ARG       # weights with nothing to write
    assert route_rc(d, w=None, probs=FAKE) == B.MOE_ERR_ARG       # probs without weights
    assert route_rc(d, host=None) == B.MOE_ERR_ARG                # eager needs the host status
    h = _handle()
    h.row_of_slot = None
    assert route_rc(d, handle=h) == B.MOE_ERR_ARG
    assert route_rc(d, idx=None) == B.MOE_ERR_ARG


def test_dispatch_pointer_rules():
    d = _desc()
    assert dispatch_rc(d, x=None) == B.MOE_ERR_ARG
    assert dispatch_rc(d, x=FAKE + 8) == B.MOE_ERR_ARG  # not 16-byte aligned
    assert dispatch_rc(d, rows=FAKE + 2) == B.MOE_ERR_ARG
    assert dispatch_rc(d, w=FAKE, row_w=None) == B.MOE_ERR_ARG
    assert dispatch_rc(d, w=None, row_w=FAKE) == B.MOE_ERR_ARG
    assert dispatch_rc(d, R=-1) == B.MOE_ERR_ARG


def test_combine_and_bwd_pointer_rules():
    d = _desc()
    assert combine_rc(d, f32=2) == B.MOE_ERR_ARG
    assert combine_rc(d, Y=None) == B.MOE_ERR_ARG
    assert combine_rc(d, out=FAKE + 4) == B.MOE_ERR_ARG
    assert bwd_rc(d, F=FAKE, dw=None) == B.MOE_ERR_ARG
    assert bwd_rc(d, F=None, dw=FAKE) == B.MOE_ERR_ARG
    assert bwd_rc(d, g=None) == B.MOE_ERR_ARG


def test_validation_agrees_with_oracle_argument_rules():
    cases = [
        dict(T=10, k=2, E=8, local_begin=0, num_local=8, pad_multiple=1),
        dict(T=10, k=2, E=8, local_begin=4, num_local=5, pad_multiple=1),
        dict(T=10, k=2, E=8, local_begin=0, num_local=8, pad_multiple=0),
        dict(T=-1, k=2, E=8, local_begin=0, num_local=8, pad_multiple=1),
        dict(T=10, k=0, E=8, local_begin=0, num_local=8, pad_multiple=1),
    ]
    for c in cases:
        want = oracle.check_args(c["T"], c["k"], c["E"], c["local_begin"], c["num_local"],
                                 c["pad_multiple"])
        d = _desc(**c)
        if want == oracle.OK:
            # valid: only the (launch-free) workspace query is called
            assert B.lib().moe_route_workspace_size(ctypes.byref(d)) > 0
        else:
            assert route_rc(d, ws_bytes=1 << 30) == want


def dbwd_rc(d, H=2048, R=10, g=FAKE, gw=None, gx=FAKE, f32=0, gtw=None):
    h = _handle()
    return B.lib().moe_dispatch_bwd(ctypes.byref(d), ctypes.byref(h), g, H, R, gw, gx, f32, gtw,
                                    None)


def test_dispatch_bwd_argument_rules():
    d = _desc()
    assert dbwd_rc(d, H=384) == B.MOE_ERR_HIDDEN
    assert dbwd_rc(d, f32=3) == B.MOE_ERR_ARG
    assert dbwd_rc(d, g=None) == B.MOE_ERR_ARG
    assert dbwd_rc(d, gx=FAKE + 2) == B.MOE_ERR_ARG
    assert dbwd_rc(d, gw=FAKE, gtw=None) == B.MOE_ERR_ARG   # weights given, nowhere to go
    assert dbwd_rc(d, gw=None, gtw=FAKE) == B.MOE_ERR_ARG   # weight grads without input
    assert "grad" in B.last_error()


def test_error_messages_are_per_thread():
    """moe_last_error belongs to the calling thread: a failure in another
    thread leaves this thread's message alone, and a new thread starts with
    none."""
    import threading

    L = B.lib()
    good = B.make_desc(100, 2, 8)
    assert L.moe_route_workspace_size(ctypes.byref(good)) > 0
    bad = B.make_desc(100, 0, 8)  # k = 0
    before = B.last_error()
    seen = {}

    def other():
        seen["fresh"] = B.last_error()
        seen["size"] = L.moe_route_workspace_size(ctypes.byref(bad))
        seen["msg"] = B.last_error()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["fresh"] == ""
    assert seen["size"] == 0 and "k must be" in seen["msg"]
    assert B.last_error() == before


@pytest.mark.skipif(__import__("torch").cuda.is_available(),
                    reason="fake device pointers: run where nothing can be launched")
def test_grids_past_2_32_work_items_are_refused():
    """A kernel dispatch packet holds the grid size in work-items as a 32-bit
    number.  A problem whose launch would need more is refused before any
    launch, with MOE_ERR_ARG and a message that says why."""
    # sync-free, 2^30 rows of H = 65536: the tail launch alone would need
    # 2^37 one-KiB pieces
    C = 1 << 30
    d = _desc(T=1000, k=2, E=8, num_local=8, pad_multiple=1, mode=B.MOE_SYNC_FREE, capacity=C)
    assert dispatch_rc(d, H=65536, R=C) == B.MOE_ERR_ARG
    assert "too large for one launch" in B.last_error()
    assert bwd_rc(d, H=65536, R=C) == B.MOE_ERR_ARG
    # 2^27 tokens of H = 65536 to combine: 2^31 workgroups
    d = _desc(T=1 << 27, k=1, E=8, num_local=8, pad_multiple=1)
    assert combine_rc(d, H=65536, R=10) == B.MOE_ERR_ARG
    assert "too large for one launch" in B.last_error()
    # the eager route-and-dispatch refuses before it launches the route
    assert rd_rc(d, H=65536) == B.MOE_ERR_ARG
    assert "too large for one launch" in B.last_error()


def rd_rc(d, H=2048, R_cap=None, idx=FAKE, w=None, probs=None, host=FAKE, x=FAKE, rows=FAKE,
          row_w=None):
    h = _handle()
    R_cap = B.lib().moe_capacity_min(ctypes.byref(d)) if R_cap is None else R_cap
    return B.lib().moe_route_dispatch(ctypes.byref(d), idx, w, probs, ctypes.byref(h), host, x, H,
                                      R_cap, rows, row_w, None, None, None)


def test_route_dispatch_argument_rules():
    """The route-and-dispatch checks the arguments of both halves before it
    launches anything, in both modes."""
    d = _desc()
    cap = B.lib().moe_capacity_min(ctypes.byref(d))
    sf = _desc(mode=B.MOE_SYNC_FREE, capacity=cap)
    # sync-free: R_cap is the capacity, the host status is not needed
    assert rd_rc(sf, R_cap=cap + 1) == B.MOE_ERR_ARG and "capacity" in B.last_error()
    assert rd_rc(sf, x=None) == B.MOE_ERR_ARG
    assert rd_rc(sf, idx=None) == B.MOE_ERR_ARG
    assert rd_rc(sf, H=384) == B.MOE_ERR_HIDDEN
    assert rd_rc(sf, w=FAKE) == B.MOE_ERR_ARG
    assert rd_rc(d, R_cap=cap - 1) == B.MOE_ERR_CAPACITY
    assert rd_rc(d, H=384) == B.MOE_ERR_HIDDEN
    assert rd_rc(d, host=None) == B.MOE_ERR_ARG
    assert rd_rc(d, x=None) == B.MOE_ERR_ARG
    assert rd_rc(d, rows=FAKE + 8) == B.MOE_ERR_ARG
    assert rd_rc(d, row_w=FAKE) == B.MOE_ERR_ARG        # row weights without topk_w
    assert rd_rc(d, probs=FAKE) == B.MOE_ERR_ARG        # probs without topk_w
    assert rd_rc(d, w=FAKE) == B.MOE_ERR_ARG            # weights with nothing to write
    assert rd_rc(_desc(k=0)) == B.MOE_ERR_ARG


def test_kernel_timer_destructor_at_interpreter_exit(monkeypatch):
    """At interpreter exit a module's globals may already be cleared when a
    KernelTimer is collected; its destructor must not raise then."""
    t = B.KernelTimer.__new__(B.KernelTimer)  # no events: nothing to destroy
    monkeypatch.setattr(B, "sys", None)
    t.__del__()
