"""Thin binding of libmoe_ceiling.so (C ABI in include/moe_ceiling.h): the
reference kernels a benchmark times beside the library's own, on the same GPU
and buffers.  Argument marshalling only; the library must have been built
(``python -m combine_topk_idx_multihot_amd.build``)."""
from __future__ import annotations

import ctypes
import os

import torch

from . import binding as _B

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libmoe_ceiling.so")

# Every symbol include/moe_ceiling.h declares.
EXPORTS = ("moe_ceiling_fill", "moe_ceiling_copy", "moe_ceiling_scatter", "moe_ceiling_gather",
           "moe_ceiling_xcd_map")
OK, ERR_ARG, ERR_HIP = 0, 1, 2

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m combine_topk_idx_multihot_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32, i64, c = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64, ctypes.c_int
        L.moe_ceiling_fill.argtypes = [vp, sz, c, vp]
        L.moe_ceiling_copy.argtypes = [vp, vp, sz, c, vp]
        L.moe_ceiling_scatter.argtypes = [vp, i64, i32, i64, i32, vp, c, vp]
        L.moe_ceiling_gather.argtypes = [vp, i64, i32, i64, i32, vp, vp, vp, c, vp]
        L.moe_ceiling_xcd_map.argtypes = [vp, i32, vp]
        for n in EXPORTS:
            getattr(L, n).restype = c
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != OK:
        raise RuntimeError(f"{what} failed with code {rc}")


def _buf(t: torch.Tensor, name: str) -> int:
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    return t.data_ptr()


def fill(dst: torch.Tensor, piece_kib: int = 1, stream=None):
    """Zero dst in address order, one wave per piece_kib KiB piece."""
    _check(lib().moe_ceiling_fill(_buf(dst, "dst"), dst.numel() * dst.element_size(), piece_kib,
                                  _B._stream(stream)), "moe_ceiling_fill")


def copy(src: torch.Tensor, dst: torch.Tensor, piece_kib: int = 1, stream=None):
    """dst[:] = src, in address order, one wave per piece_kib KiB piece."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst is smaller than src")
    _check(lib().moe_ceiling_copy(_buf(src, "src"), _buf(dst, "dst"), n, piece_kib,
                                  _B._stream(stream)), "moe_ceiling_copy")


def scatter(row_of_slot: torch.Tensor, rows: torch.Tensor, seg_kib: int = 1, stream=None):
    """Zero every row of rows [R,H] bf16 that row_of_slot [T,k] int32 names,
    token-major, one workgroup per token (the dispatch's store pattern without
    its reads)."""
    if row_of_slot.dtype != torch.int32 or row_of_slot.dim() != 2 or rows.dim() != 2:
        raise ValueError("row_of_slot must be [T,k] int32 and rows [R,H]")
    T, k = row_of_slot.shape
    R, H = rows.shape
    _check(lib().moe_ceiling_scatter(_buf(row_of_slot, "row_of_slot"), T, k, R, H,
                                     _buf(rows, "rows"), seg_kib, _B._stream(stream)),
           "moe_ceiling_scatter")


def gather(row_of_slot: torch.Tensor, Y: torch.Tensor, out: torch.Tensor | None = None,
           sink: torch.Tensor | None = None, seg_kib: int = 2, stream=None):
    """The combine's reads: each token's rows of Y [R,H] bf16 that
    row_of_slot [T,k] int32 names, summed in fp32; the sums stored into out
    [T,H] bf16 (truncated), or, with out None, nothing stored (read only; sink
    is a one-word int32 GPU tensor)."""
    if row_of_slot.dtype != torch.int32 or row_of_slot.dim() != 2 or Y.dim() != 2:
        raise ValueError("row_of_slot must be [T,k] int32 and Y [R,H]")
    T, k = row_of_slot.shape
    R, H = Y.shape
    if out is not None and (out.dim() != 2 or out.shape[0] < T or out.shape[1] != H):
        raise ValueError("out must be [T,H]")
    if out is None and (sink is None or sink.numel() < 1):
        raise ValueError("a read-only gather needs a sink word")
    _check(lib().moe_ceiling_gather(_buf(row_of_slot, "row_of_slot"), T, k, R, H, _buf(Y, "Y"),
                                    None if out is None else _buf(out, "out"),
                                    None if sink is None else _buf(sink, "sink"), seg_kib,
                                    _B._stream(stream)), "moe_ceiling_gather")


def xcd_map(nblocks: int = 4096, stream=None) -> torch.Tensor:
    """The XCD each of `nblocks` workgroups ran on (int32 on the GPU)."""
    out = torch.full((nblocks,), -1, dtype=torch.int32, device="cuda")
    _check(lib().moe_ceiling_xcd_map(_buf(out, "out"), nblocks, _B._stream(stream)),
           "moe_ceiling_xcd_map")
    return out


def xcd_round_robin(nblocks: int = 4096) -> dict:
    """Whether workgroup j ran on XCD j mod (number of XCDs seen), as the
    library's row kernels assume."""
    m = xcd_map(nblocks).cpu().numpy()
    n = len(set(m.tolist()))
    j = list(range(nblocks))
    match = sum(1 for i in j if m[i] == i % n) / nblocks
    return {"xcds_seen": n, "blocks": nblocks, "frac_j_mod_xcds": round(match, 4)}
