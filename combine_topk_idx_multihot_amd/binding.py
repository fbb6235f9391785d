"""Thin Python binding of libmoe_mi355x (C ABI in include/moe_mi355x.h).

Argument marshalling only: torch supplies device memory and streams, every step
of the path runs in the library's HIP kernels.  The ``moe_*`` functions mirror
the C entry points one for one; before passing a pointer they check that each
tensor lives on the GPU, is contiguous, has the expected dtype and is large
enough for what the call will write (the C ABI takes plain pointers and cannot).
The convenience functions at the bottom (``alloc_handle``, ``route``,
``dispatch``, ``dispatch_fp8``, ``combine``, ``combine_bwd``, ``dispatch_bwd``)
only add output allocation.  ``PreparedDispatch``, ``PreparedCombine`` and
``PreparedCombineBwd`` check reused buffers once and then take only the step's
row count; ``KernelTimer`` times one call's kernels.

The library is loaded on first use; if it has not been built this raises
(there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
import sys
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libmoe_mi355x.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_HIDDEN, MOE_ERR_CAPACITY = 0, 1, 2, 3
MOE_ERR_WORKSPACE, MOE_ERR_INDEX, MOE_ERR_HIP, MOE_ERR_DEVICE = 4, 5, 6, 7
MOE_EAGER, MOE_SYNC_FREE = 0, 1
MOE_FLAG_BAD_ID, MOE_FLAG_DUPLICATE, MOE_FLAG_ROWS_MISMATCH = 1, 2, 4
MOE_NOALLOC_SCRATCH_BYTES = 4194304  # the fixed route scratch of moe_route_build_noalloc

# Every symbol include/moe_mi355x.h declares.
EXPORTS = ("moe_capacity_min", "moe_route_workspace_size", "moe_route_build",
           "moe_route_build_noalloc", "moe_route_dispatch", "moe_dispatch",
           "moe_dispatch_fp8", "moe_combine", "moe_combine_bwd", "moe_dispatch_bwd",
           "moe_last_error", "moe_device_check", "moe_time_next_call")


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[moe status {code}] {msg}")
        self.code = code


class Desc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("k", ctypes.c_int32), ("E", ctypes.c_int32),
                ("local_begin", ctypes.c_int32), ("num_local", ctypes.c_int32),
                ("pad_multiple", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("idx_is_i64", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("capacity", ctypes.c_int64)]


class _Handle(ctypes.Structure):
    _fields_ = [("routing_map", ctypes.c_void_p), ("tokens_per_expert", ctypes.c_void_p),
                ("padded_offsets", ctypes.c_void_p), ("row_of_slot", ctypes.c_void_p),
                ("status", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe_mi355x.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m combine_topk_idx_multihot_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        pd, ph = ctypes.POINTER(Desc), ctypes.POINTER(_Handle)
        L.moe_capacity_min.argtypes = [pd]
        L.moe_capacity_min.restype = i64
        L.moe_route_workspace_size.argtypes = [pd]
        L.moe_route_workspace_size.restype = ctypes.c_size_t
        L.moe_route_build.argtypes = [pd, vp, vp, vp, ph, vp, vp]
        L.moe_route_build.restype = ctypes.c_int
        L.moe_route_build_noalloc.argtypes = [pd, vp, vp, vp, ph, vp, vp]
        L.moe_route_build_noalloc.restype = ctypes.c_int
        L.moe_dispatch.argtypes = [pd, ph, vp, i32, vp, i64, vp, vp, vp, vp, vp]
        L.moe_dispatch.restype = ctypes.c_int
        L.moe_dispatch_fp8.argtypes = [pd, ph, vp, i32, vp, i64, vp, vp, vp, vp, vp, vp]
        L.moe_dispatch_fp8.restype = ctypes.c_int
        L.moe_combine.argtypes = [pd, ph, vp, i32, i64, vp, i32, vp]
        L.moe_combine.restype = ctypes.c_int
        L.moe_combine_bwd.argtypes = [pd, ph, vp, vp, i32, i64, vp, vp, vp]
        L.moe_combine_bwd.restype = ctypes.c_int
        L.moe_dispatch_bwd.argtypes = [pd, ph, vp, i32, i64, vp, vp, i32, vp, vp]
        L.moe_dispatch_bwd.restype = ctypes.c_int
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_device_check.argtypes = [ctypes.c_int]
        L.moe_device_check.restype = ctypes.c_int
        L.moe_route_dispatch.argtypes = [pd, vp, vp, vp, ph, vp, vp, i32, i64, vp, vp, vp, vp, vp]
        L.moe_route_dispatch.restype = ctypes.c_int
        L.moe_time_next_call.argtypes = [vp, vp]
        L.moe_time_next_call.restype = ctypes.c_int
        _lib = L
    return _lib


def last_error() -> str:
    return lib().moe_last_error().decode()


def _check(rc: int):
    if rc != MOE_OK:
        raise MoeError(rc, last_error())
    return rc


def make_desc(T: int, k: int, E: int, local_begin: int = 0, num_local: int | None = None,
              pad_multiple: int = 1, mode: int = MOE_EAGER, idx_is_i64: bool = False,
              capacity: int = 0) -> Desc:
    return Desc(T=T, k=k, E=E, local_begin=local_begin,
                num_local=E if num_local is None else num_local, pad_multiple=pad_multiple,
                mode=mode, idx_is_i64=int(bool(idx_is_i64)), reserved=0, capacity=capacity)


# ---------------------------------------------------------------------------
# tensor checks (the C ABI cannot see buffer sizes)
# ---------------------------------------------------------------------------

def _dev(t: torch.Tensor | None, name: str, dtype, numel: int, optional: bool = False):
    if t is None:
        if optional:
            return None
        raise MoeError(MOE_ERR_ARG, f"{name} is required")
    try:
        ok = t.is_cuda and t.dtype in dtype and t.is_contiguous() and t.numel() >= numel
    except (AttributeError, TypeError):
        ok = False
    if not ok:
        _explain(t, name, dtype, numel)
    return t.data_ptr()


def _explain(t, name, dtype, numel):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise MoeError(MOE_ERR_ARG, f"{name} must be a GPU tensor")
    if t.dtype not in dtype:
        raise MoeError(MOE_ERR_ARG, f"{name} has dtype {t.dtype}, expected one of {dtype}")
    if not t.is_contiguous():
        raise MoeError(MOE_ERR_ARG, f"{name} must be contiguous")
    raise MoeError(MOE_ERR_ARG, f"{name} has {t.numel()} elements, needs {numel}")


# dtype sets accepted by _dev
_U8, _I32, _I64, _F32, _BF16 = ((torch.uint8,), (torch.int32,), (torch.int64,), (torch.float32,),
                                (torch.bfloat16,))


# torch's raw current-stream query skips building a Stream object (a few
# microseconds per call); it is not public API, so the public query stands in
# where a torch build lacks it.
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> int:
    if stream is None:
        if _raw_current_stream is not None:
            return _raw_current_stream(torch.cuda.current_device())
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


@dataclass
class Handle:
    """Dispatch handle: plain device tensors plus a pinned host status."""
    desc: Desc
    routing_map: torch.Tensor | None   # [T,E] uint8
    tokens_per_expert: torch.Tensor    # [EL] int32
    padded_offsets: torch.Tensor       # [EL+1] int32
    row_of_slot: torch.Tensor          # [T,k] int32
    status: torch.Tensor               # [4] int32 (device)
    host_status: torch.Tensor          # [4] int32 (pinned host)
    workspace: torch.Tensor | None     # [moe_route_workspace_size] uint8 (device): the
                                       # route's scratch and, for dense routing, its row
                                       # list, which dispatch and combine_bwd walk

    def c(self) -> _Handle:
        """The C struct, checked and built once: a Handle's tensors are not to
        be reassigned after creation (build a new Handle instead)."""
        cs = self.__dict__.get("_cstruct")
        if cs is not None:
            return cs
        d = self.desc
        ws = self.workspace
        cs = _Handle(
            workspace=None if ws is None else _dev(ws, "workspace", _U8,
                                                   moe_route_workspace_size(d)),
            workspace_bytes=0 if ws is None else ws.numel(),
            routing_map=_dev(self.routing_map, "routing_map", _U8, d.T * d.E, True),
            tokens_per_expert=_dev(self.tokens_per_expert, "tokens_per_expert", _I32, d.num_local),
            padded_offsets=_dev(self.padded_offsets, "padded_offsets", _I32, d.num_local + 1),
            row_of_slot=_dev(self.row_of_slot, "row_of_slot", _I32, d.T * d.k),
            status=_dev(self.status, "status", _I32, 4))
        hs = self.host_status
        if hs.is_cuda or hs.dtype != torch.int32 or hs.numel() < 4 or not hs.is_contiguous():
            raise MoeError(MOE_ERR_ARG, "host_status must be a host int32 tensor of 4 elements")
        self.__dict__["_cstruct"] = cs
        self.__dict__["_cref"] = ctypes.byref(cs)
        return cs

    def cref(self):
        self.c()
        return self.__dict__["_cref"]

    def _host_words(self):
        hw = self.__dict__.get("_host_np")
        if hw is None:
            hw = self.__dict__["_host_np"] = self.host_status.numpy()
        return hw

    @property
    def total(self) -> int:
        """Padded row total from the last eager moe_route_build."""
        return int(self._host_words()[0])

    @property
    def flags(self) -> int:
        return int(self._host_words()[1])


def alloc_handle(desc: Desc, device="cuda", with_map: bool = True,
                 with_workspace: bool = True) -> Handle:
    """Handle tensors for `desc`; with_workspace=False leaves the route
    workspace out, as moe_route_build_noalloc requires."""
    T, E, EL, k = desc.T, desc.E, desc.num_local, desc.k
    return Handle(
        desc=desc,
        routing_map=torch.empty((T, E), dtype=torch.uint8, device=device) if with_map else None,
        tokens_per_expert=torch.empty(EL, dtype=torch.int32, device=device),
        padded_offsets=torch.empty(EL + 1, dtype=torch.int32, device=device),
        row_of_slot=torch.empty((T, k), dtype=torch.int32, device=device),
        status=torch.empty(4, dtype=torch.int32, device=device),
        host_status=torch.zeros(4, dtype=torch.int32, pin_memory=True),
        workspace=(torch.empty(moe_route_workspace_size(desc), dtype=torch.uint8, device=device)
                   if with_workspace else None))


# ---------------------------------------------------------------------------
# the C entry points, one for one
# ---------------------------------------------------------------------------

def moe_capacity_min(desc: Desc) -> int:
    return int(lib().moe_capacity_min(ctypes.byref(desc)))


def moe_route_workspace_size(desc: Desc) -> int:
    n = int(lib().moe_route_workspace_size(ctypes.byref(desc)))
    if n == 0:
        raise MoeError(MOE_ERR_ARG, last_error())
    return n


def moe_route_build(desc: Desc, topk_idx: torch.Tensor, handle: Handle,
                    topk_w: torch.Tensor | None = None, multihot_probs: torch.Tensor | None = None,
                    stream=None) -> int:
    """Returns MOE_OK; eager mode fills handle.host_status (total, flags, data rows)."""
    n = desc.T * desc.k
    p_idx = _dev(topk_idx, "topk_idx", _I64 if desc.idx_is_i64 else _I32, n) if n else None
    p_w = _dev(topk_w, "topk_w", _F32, n, optional=True)
    p_probs = _dev(multihot_probs, "multihot_probs", _F32, desc.T * desc.E, optional=True)
    href = handle.cref()
    return _check(lib().moe_route_build(ctypes.byref(desc), p_idx, p_w, p_probs, href,
                                        handle.host_status.data_ptr(), _stream(stream)))


def moe_route_build_noalloc(desc: Desc, topk_idx: torch.Tensor, handle: Handle,
                            topk_w: torch.Tensor | None = None,
                            multihot_probs: torch.Tensor | None = None, stream=None) -> int:
    """moe_route_build with the route's scratch in the library's fixed per-GPU
    array: the handle must have no workspace (alloc_handle(...,
    with_workspace=False)).  Nothing is allocated by the call."""
    n = desc.T * desc.k
    p_idx = _dev(topk_idx, "topk_idx", _I64 if desc.idx_is_i64 else _I32, n) if n else None
    p_w = _dev(topk_w, "topk_w", _F32, n, optional=True)
    p_probs = _dev(multihot_probs, "multihot_probs", _F32, desc.T * desc.E, optional=True)
    return _check(lib().moe_route_build_noalloc(ctypes.byref(desc), p_idx, p_w, p_probs,
                                                handle.cref(), handle.host_status.data_ptr(),
                                                _stream(stream)))


def moe_route_dispatch(desc: Desc, topk_idx: torch.Tensor, handle: Handle, x: torch.Tensor,
                       H: int, rows: torch.Tensor, topk_w: torch.Tensor | None = None,
                       multihot_probs: torch.Tensor | None = None,
                       row_w: torch.Tensor | None = None, row_token: torch.Tensor | None = None,
                       row_expert: torch.Tensor | None = None, stream=None) -> int:
    """Route and dispatch in one call into buffers of R_cap = rows.shape[0]
    rows.  Eager: R_cap >= moe_capacity_min, the dispatch is queued before
    the row count is read back; handle.total is then the count and rows
    [0, total) are filled.  Sync-free: R_cap = desc.capacity, nothing waits,
    every row is written; a decode-sized route runs in the dispatch's own
    launch."""
    T, k = desc.T, desc.k
    R_cap = rows.numel() // H if H > 0 else 0
    p_idx = _dev(topk_idx, "topk_idx", _I64 if desc.idx_is_i64 else _I32, T * k) if T * k else None
    p_w = _dev(topk_w, "topk_w", _F32, T * k, optional=True) if T else None
    p_probs = _dev(multihot_probs, "multihot_probs", _F32, T * desc.E, optional=True)
    p_x = _dev(x, "x", _BF16, T * H) if T else None
    p_rows = _dev(rows, "rows", _BF16, R_cap * H) if R_cap else None
    p_rw = _dev(row_w, "row_w", _F32, R_cap, optional=True)
    p_rt = _dev(row_token, "row_token", _I32, R_cap, optional=True)
    p_re = _dev(row_expert, "row_expert", _I32, R_cap, optional=True)
    return _check(lib().moe_route_dispatch(ctypes.byref(desc), p_idx, p_w, p_probs, handle.cref(),
                                           handle.host_status.data_ptr(), p_x, H, R_cap, p_rows,
                                           p_rw, p_rt, p_re, _stream(stream)))


def moe_dispatch(desc: Desc, handle: Handle, x: torch.Tensor, H: int, R: int, rows: torch.Tensor,
                 topk_w: torch.Tensor | None = None, row_w: torch.Tensor | None = None,
                 row_token: torch.Tensor | None = None, row_expert: torch.Tensor | None = None,
                 stream=None) -> int:
    p_x = _dev(x, "x", _BF16, desc.T * H) if desc.T else None
    p_rows = _dev(rows, "rows", _BF16, R * H) if R else None
    p_w = _dev(topk_w, "topk_w", _F32, desc.T * desc.k, optional=True)
    p_rw = _dev(row_w, "row_w", _F32, R, optional=True)
    if desc.T == 0:
        p_w = None
    if R == 0:
        p_rw = None
        if p_w is not None:  # no row to weight; the C ABI pairs the two pointers
            p_w = None
    p_rt = _dev(row_token, "row_token", _I32, R, optional=True)
    p_re = _dev(row_expert, "row_expert", _I32, R, optional=True)
    return _check(lib().moe_dispatch(ctypes.byref(desc), handle.cref(), p_x, H, p_w, R, p_rows,
                                     p_rw, p_rt, p_re, _stream(stream)))


class PreparedDispatch:
    """moe_dispatch over buffers that a loop reuses on every step, checked once.

    For eager loops whose row buffers are sized for the worst case (for
    instance moe_capacity_min rows): each call passes only the step's row count
    R (the host total from that step's moe_route_build) and fills rows [0, R).
    The Python-side checks of moe_dispatch are made here once, against the
    buffers' capacity, which takes them off the path between the eager
    readback and the dispatch launch; the library still checks every argument
    on every call.  The tensors must stay as they are (no resize_ or set_)
    while the object is in use; it holds references to them.
    """

    def __init__(self, desc: Desc, handle: Handle, x: torch.Tensor, H: int, rows: torch.Tensor,
                 topk_w: torch.Tensor | None = None, row_w: torch.Tensor | None = None,
                 row_token: torch.Tensor | None = None, row_expert: torch.Tensor | None = None,
                 stream=None):
        if H <= 0 or rows is None:
            raise MoeError(MOE_ERR_ARG, "H must be positive and rows given")
        cap = rows.numel() // H
        if cap == 0:
            raise MoeError(MOE_ERR_ARG, "rows holds no [H] row")
        if (topk_w is None) != (row_w is None):
            raise MoeError(MOE_ERR_ARG, "topk_w and row_w go together")
        p_x = _dev(x, "x", _BF16, desc.T * H) if desc.T else None
        p_rows = _dev(rows, "rows", _BF16, cap * H)
        p_w = _dev(topk_w, "topk_w", _F32, desc.T * desc.k, optional=True) if desc.T else None
        p_rw = _dev(row_w, "row_w", _F32, cap, optional=True) if p_w is not None else None
        p_rt = _dev(row_token, "row_token", _I32, cap, optional=True)
        p_re = _dev(row_expert, "row_expert", _I32, cap, optional=True)
        self.capacity = cap
        self._fn = lib().moe_dispatch
        # a private copy: the checks above hold for this descriptor, whatever
        # later becomes of the caller's
        self._desc = Desc.from_buffer_copy(desc)
        self._head = (ctypes.byref(self._desc), handle.cref(), p_x, H, p_w)
        self._tail = (p_rows, p_rw, p_rt, p_re, _stream(stream))
        self._keep = (handle, x, rows, topk_w, row_w, row_token, row_expert)

    def __call__(self, R: int) -> int:
        if not 0 <= R <= self.capacity:
            raise MoeError(MOE_ERR_ARG, f"R={R} outside [0, {self.capacity}] rows of the buffers")
        return _check(self._fn(*self._head, R, *self._tail))



class PreparedCombine:
    """moe_combine over buffers that a loop reuses on every step, checked once.

    Y holds up to `capacity` rows of H (for instance the experts' output
    buffer sized for the worst case); each call passes only the step's row
    count R and combines rows [0, R) into `out`.  As with PreparedDispatch,
    the Python-side checks are made here once, which takes them off the path
    between the eager readback and the launch; the library still checks every
    argument on every call.  The tensors must stay as they are while the
    object is in use; it holds references to them.
    """

    def __init__(self, desc: Desc, handle: Handle, Y: torch.Tensor, H: int, out: torch.Tensor,
                 stream=None):
        if H <= 0 or Y is None:
            raise MoeError(MOE_ERR_ARG, "H must be positive and Y given")
        cap = Y.numel() // H
        p_y = _dev(Y, "Y", _BF16, cap * H) if cap else None
        p_o = _dev(out, "out", (torch.bfloat16, torch.float32), desc.T * H) if desc.T else None
        self.capacity = cap
        self._fn = lib().moe_combine
        self._desc = Desc.from_buffer_copy(desc)
        self._head = (ctypes.byref(self._desc), handle.cref(), p_y, H)
        self._tail = (p_o, int(out.dtype == torch.float32), _stream(stream))
        self._keep = (handle, Y, out)

    def __call__(self, R: int) -> int:
        if not 0 <= R <= self.capacity:
            raise MoeError(MOE_ERR_ARG, f"R={R} outside [0, {self.capacity}] rows of the buffers")
        return _check(self._fn(*self._head, R, *self._tail))


class PreparedCombineBwd:
    """moe_combine_bwd over buffers that a loop reuses on every step, checked
    once: grad_rows (and expert_out, when dw is wanted) hold up to `capacity`
    rows; each call passes only the step's row count R.  Same contract as
    PreparedCombine."""

    def __init__(self, desc: Desc, handle: Handle, grad_out: torch.Tensor, H: int,
                 grad_rows: torch.Tensor, expert_out: torch.Tensor | None = None,
                 dw: torch.Tensor | None = None, stream=None):
        if H <= 0 or grad_rows is None:
            raise MoeError(MOE_ERR_ARG, "H must be positive and grad_rows given")
        if (expert_out is None) != (dw is None):
            raise MoeError(MOE_ERR_ARG, "expert_out and dw go together")
        cap = grad_rows.numel() // H
        if expert_out is not None:
            cap = min(cap, expert_out.numel() // H)
        p_g = _dev(grad_out, "grad_out", _BF16, desc.T * H) if desc.T else None
        p_gr = _dev(grad_rows, "grad_rows", _BF16, cap * H) if cap else None
        p_f = _dev(expert_out, "expert_out", _BF16, cap * H, optional=True) if cap else None
        p_dw = _dev(dw, "dw", _F32, desc.T * desc.k, optional=True) if p_f is not None else None
        if desc.T == 0:  # no slot: nothing for dw to hold, expert_out is not read
            p_f = p_dw = None
        self.capacity = cap
        self._fn = lib().moe_combine_bwd
        self._desc = Desc.from_buffer_copy(desc)
        self._head = (ctypes.byref(self._desc), handle.cref(), p_g, p_f, H)
        self._tail = (p_gr, p_dw, _stream(stream))
        self._keep = (handle, grad_out, grad_rows, expert_out, dw)

    def __call__(self, R: int) -> int:
        if not 0 <= R <= self.capacity:
            raise MoeError(MOE_ERR_ARG, f"R={R} outside [0, {self.capacity}] rows of the buffers")
        return _check(self._fn(*self._head, R, *self._tail))

def moe_dispatch_fp8(desc: Desc, handle: Handle, x: torch.Tensor, H: int, R: int,
                     rows_q: torch.Tensor, row_scale: torch.Tensor,
                     topk_w: torch.Tensor | None = None, row_w: torch.Tensor | None = None,
                     row_token: torch.Tensor | None = None, row_expert: torch.Tensor | None = None,
                     stream=None) -> int:
    p_x = _dev(x, "x", _BF16, desc.T * H) if desc.T else None
    p_q = _dev(rows_q, "rows_q", (torch.uint8, torch.float8_e4m3fn), R * H) if R else None
    p_s = _dev(row_scale, "row_scale", _F32, R * (H // 128)) if R else None
    p_w = _dev(topk_w, "topk_w", _F32, desc.T * desc.k, optional=True)
    p_rw = _dev(row_w, "row_w", _F32, R, optional=True)
    if desc.T == 0:
        p_w = None
    if R == 0:
        p_rw = None
        if p_w is not None:
            p_w = None
    p_rt = _dev(row_token, "row_token", _I32, R, optional=True)
    p_re = _dev(row_expert, "row_expert", _I32, R, optional=True)
    return _check(lib().moe_dispatch_fp8(ctypes.byref(desc), handle.cref(), p_x, H, p_w, R, p_q,
                                         p_s, p_rw, p_rt, p_re, _stream(stream)))


def moe_combine(desc: Desc, handle: Handle, Y: torch.Tensor, H: int, R: int, out: torch.Tensor,
                stream=None) -> int:
    out_f32 = out.dtype == torch.float32
    p_y = _dev(Y, "Y", _BF16, R * H) if R else None
    p_o = _dev(out, "out", (torch.bfloat16, torch.float32), desc.T * H) if desc.T else None
    return _check(lib().moe_combine(ctypes.byref(desc), handle.cref(), p_y, H, R, p_o,
                                    int(out_f32), _stream(stream)))


def moe_combine_bwd(desc: Desc, handle: Handle, grad_out: torch.Tensor, H: int, R: int,
                    grad_rows: torch.Tensor, expert_out: torch.Tensor | None = None,
                    dw: torch.Tensor | None = None, stream=None) -> int:
    p_g = _dev(grad_out, "grad_out", _BF16, desc.T * H) if desc.T else None
    p_gr = _dev(grad_rows, "grad_rows", _BF16, R * H) if R else None
    p_f = _dev(expert_out, "expert_out", _BF16, R * H, optional=True) if R else None
    p_dw = _dev(dw, "dw", _F32, desc.T * desc.k, optional=True)
    if desc.T == 0:  # no slot: nothing for dw to hold, expert_out is not read
        p_f = p_dw = None
    return _check(lib().moe_combine_bwd(ctypes.byref(desc), handle.cref(), p_g, p_f, H, R, p_gr,
                                        p_dw, _stream(stream)))


def moe_dispatch_bwd(desc: Desc, handle: Handle, grad_rows: torch.Tensor, H: int, R: int,
                     grad_x: torch.Tensor, grad_row_w: torch.Tensor | None = None,
                     grad_topk_w: torch.Tensor | None = None, stream=None) -> int:
    f32 = grad_x.dtype == torch.float32
    p_g = _dev(grad_rows, "grad_rows", _BF16, R * H) if R else None
    p_x = _dev(grad_x, "grad_x", (torch.bfloat16, torch.float32), desc.T * H) if desc.T else None
    p_rw = _dev(grad_row_w, "grad_row_w", _F32, R, optional=True) if R else None
    p_tw = _dev(grad_topk_w, "grad_topk_w", _F32, desc.T * desc.k, optional=True)
    if desc.T == 0:
        p_tw = None
    if p_tw is None:
        p_rw = None
    return _check(lib().moe_dispatch_bwd(ctypes.byref(desc), handle.cref(), p_g, H, R, p_rw, p_x,
                                         int(f32), p_tw, _stream(stream)))


def moe_device_check(device: int = 0) -> int:
    return _check(lib().moe_device_check(device))


def _event(ev) -> int | None:
    if ev is None:
        return None
    if isinstance(ev, torch.cuda.Event):
        if not ev.cuda_event:
            raise MoeError(MOE_ERR_ARG, "the torch event has no HIP event yet: record it once first")
        return ev.cuda_event
    return int(ev)


def moe_time_next_call(start_event=None, stop_event=None) -> int:
    """The next library call on this thread times its kernels into the two
    events (torch.cuda.Event with enable_timing=True, recorded once so that
    its HIP event exists, or raw hipEvent_t handles)."""
    return _check(lib().moe_time_next_call(_event(start_event), _event(stop_event)))


_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hip_runtime_api.h


class KernelTimer:
    """Two HIP events for moe_time_next_call, created with
    hipEventDisableSystemFence: events used only for timing need no
    system-scope cache write-back when they complete, which otherwise delays
    the next kernel by a few microseconds.  The events come from the HIP
    runtime the library itself is linked against.

        t = KernelTimer(stream)
        t.arm(); B.moe_combine_bwd(...)       # the next call is timed
        torch.cuda.synchronize(); t.elapsed_ms()
    """

    def __init__(self, stream=None):
        L = lib()
        if not getattr(L, "_timer_protos", False):
            L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            L.hipEventDestroy.argtypes = [ctypes.c_void_p]
            L._timer_protos = True
        self._L = L
        self.start = self._create()
        self.stop = self._create()
        s = _stream(stream)
        for e in (self.start, self.stop):  # so that elapsed_ms is defined from the start
            self._hip(L.hipEventRecord(e, s), "hipEventRecord")

    def _hip(self, rc, what):
        if rc != 0:
            raise MoeError(MOE_ERR_HIP, f"{what} failed with HIP error {rc}")

    def _create(self):
        e = ctypes.c_void_p()
        self._hip(self._L.hipEventCreateWithFlags(ctypes.byref(e), _HIP_EVENT_DISABLE_SYSTEM_FENCE),
                  "hipEventCreateWithFlags")
        return e.value

    def arm(self):
        """Time the kernels of the next library call made on this thread."""
        _check(self._L.moe_time_next_call(self.start, self.stop))

    def elapsed_ms(self) -> float:
        """Device time of the timed call's kernels; valid once they are done."""
        f = ctypes.c_float()
        self._hip(self._L.hipEventElapsedTime(ctypes.byref(f), self.start, self.stop),
                  "hipEventElapsedTime")
        return f.value

    def since_ms(self, earlier: "KernelTimer") -> float:
        """Device time from the start of `earlier`'s timed call to the start
        of this one's (both done): for the same call in consecutive steps,
        the device time of one whole step."""
        f = ctypes.c_float()
        self._hip(self._L.hipEventElapsedTime(ctypes.byref(f), earlier.start, self.start),
                  "hipEventElapsedTime")
        return f.value

    def close(self):
        for name in ("start", "stop"):
            e = self.__dict__.pop(name, None)
            if e:
                self._L.hipEventDestroy(e)

    def __del__(self, _finalizing=sys.is_finalizing):
        # bound at definition: at interpreter exit this module's globals (sys
        # among them) may already be gone, and the HIP runtime torn down
        if _finalizing():
            return
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------------------
# convenience wrappers that allocate outputs
# ---------------------------------------------------------------------------

def route(desc: Desc, topk_idx: torch.Tensor, topk_w: torch.Tensor | None = None,
          want_probs: bool = False, with_map: bool = True, handle: Handle | None = None,
          stream=None):
    """moe_route_build with fresh outputs.  Returns (handle, multihot_probs or None)."""
    dev = topk_idx.device
    handle = handle or alloc_handle(desc, dev, with_map=with_map)
    probs = torch.empty((desc.T, desc.E), dtype=torch.float32, device=dev) if want_probs else None
    moe_route_build(desc, topk_idx, handle, topk_w if want_probs else None, probs, stream=stream)
    return handle, probs


def rows_for(desc: Desc, handle: Handle) -> int:
    return desc.capacity if desc.mode == MOE_SYNC_FREE else handle.total


def dispatch(desc: Desc, handle: Handle, x: torch.Tensor, topk_w: torch.Tensor | None = None,
             meta: bool = True, stream=None):
    """moe_dispatch with fresh outputs: (rows, row_w, row_token, row_expert)."""
    R, H, dev = rows_for(desc, handle), x.shape[1], x.device
    rows = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    row_w = torch.empty(R, dtype=torch.float32, device=dev) if topk_w is not None else None
    rt = torch.empty(R, dtype=torch.int32, device=dev) if meta else None
    re = torch.empty(R, dtype=torch.int32, device=dev) if meta else None
    moe_dispatch(desc, handle, x, H, R, rows, topk_w, row_w, rt, re, stream=stream)
    return rows, row_w, rt, re


def dispatch_fp8(desc: Desc, handle: Handle, x: torch.Tensor, topk_w: torch.Tensor | None = None,
                 meta: bool = True, stream=None):
    """moe_dispatch_fp8 with fresh outputs: (rows_q [R,H] float8_e4m3fn, row_scale [R,H/128],
    row_w, row_token, row_expert)."""
    R, H, dev = rows_for(desc, handle), x.shape[1], x.device
    rows_q = torch.empty((R, H), dtype=torch.float8_e4m3fn, device=dev)
    row_scale = torch.empty((R, H // 128), dtype=torch.float32, device=dev)
    row_w = torch.empty(R, dtype=torch.float32, device=dev) if topk_w is not None else None
    rt = torch.empty(R, dtype=torch.int32, device=dev) if meta else None
    re = torch.empty(R, dtype=torch.int32, device=dev) if meta else None
    moe_dispatch_fp8(desc, handle, x, H, R, rows_q, row_scale, topk_w, row_w, rt, re,
                     stream=stream)
    return rows_q, row_scale, row_w, rt, re


def combine(desc: Desc, handle: Handle, Y: torch.Tensor, out_dtype=torch.bfloat16, stream=None):
    R, H = Y.shape
    out = torch.empty((desc.T, H), dtype=out_dtype, device=Y.device)
    moe_combine(desc, handle, Y, H, R, out, stream=stream)
    return out


def combine_bwd(desc: Desc, handle: Handle, grad_out: torch.Tensor, R: int,
                expert_out: torch.Tensor | None = None, stream=None):
    H, dev = grad_out.shape[1], grad_out.device
    grad_rows = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((desc.T, desc.k), dtype=torch.float32, device=dev) if expert_out is not None else None
    moe_combine_bwd(desc, handle, grad_out, H, R, grad_rows, expert_out, dw, stream=stream)
    return grad_rows, dw


def dispatch_bwd(desc: Desc, handle: Handle, grad_rows: torch.Tensor,
                 grad_row_w: torch.Tensor | None = None, out_dtype=torch.bfloat16, stream=None):
    """moe_dispatch_bwd with fresh outputs: (grad_x, grad_topk_w or None)."""
    R, H = grad_rows.shape
    gx = torch.empty((desc.T, H), dtype=out_dtype, device=grad_rows.device)
    gtw = (torch.empty((desc.T, desc.k), dtype=torch.float32, device=grad_rows.device)
           if grad_row_w is not None else None)
    moe_dispatch_bwd(desc, handle, grad_rows, H, R, gx, grad_row_w, gtw, stream=stream)
    return gx, gtw
