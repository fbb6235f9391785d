"""Oracle for the MoE routing / dispatch / combine path -- TEST INFRASTRUCTURE ONLY.

This package wraps ``moe_oracle.c`` (plain single-threaded C, built with gcc) with
numpy in and numpy out.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it; the GPU library never does, and the oracle never
imports the GPU library.

What it computes, and the readings it takes where the pages are silent, is
documented at the top of ``moe_oracle.c``.  Sources: "feat: add hybridep"
(Changelog; review of the dispatch hunk and of ``_indices_to_multihot``) and
"Add the deepep expert-parallel implementation" ("What this adds": Expanded
layout, Eager vs captured, Custom ops, Training; requirements paragraph).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Return codes of the oracle (its own statement of the error contract).
OK, ERR_ARG, ERR_HIDDEN, ERR_CAPACITY, ERR_INDEX = 0, 1, 2, 3, 5
FLAG_BAD_ID, FLAG_DUP = 1, 2


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile moe_oracle.c into liboracle.so with gcc (strict IEEE: no
    contraction of a*b+c into fma, no fast-math)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        # MOE_ORACLE_LIB: load another build of this source instead (the
        # planted-mistake test points it at deliberately broken copies)
        path = os.environ.get("MOE_ORACLE_LIB")
        if path is None:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        L = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        L.oracle_bf16_round.argtypes = [ctypes.c_float]
        L.oracle_bf16_round.restype = ctypes.c_uint16
        L.oracle_bf16_round_array.argtypes = [vp, vp, i64]
        L.oracle_bf16_round_array.restype = None
        L.oracle_capacity_min.argtypes = [i64, i32, i32, i32]
        L.oracle_capacity_min.restype = i64
        L.oracle_check_args.argtypes = [i64, i32, i32, i32, i32, i32, i32, i64]
        L.oracle_check_args.restype = ctypes.c_int
        L.oracle_check_hidden.argtypes = [i64]
        L.oracle_check_hidden.restype = ctypes.c_int
        L.oracle_route.argtypes = ([i64, i32, i32, i32, i32, i32, i32, i64]
                                   + [vp, vp, vp, i64]
                                   + [vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp])
        L.oracle_route.restype = ctypes.c_int
        L.oracle_combine.argtypes = [i64, i32, i32, i32, i32, vp, vp, i64, i64, vp, vp, vp]
        L.oracle_combine.restype = ctypes.c_int
        L.oracle_combine_bwd.argtypes = [i64, i32, i32, i32, i32, vp, vp, vp, i64, i64,
                                         vp, vp, vp, vp]
        L.oracle_combine_bwd.restype = ctypes.c_int
        L.oracle_dispatch_bwd.argtypes = [i64, i32, i32, i32, i32, vp, vp, i64, i64, vp, vp, vp,
                                          vp, vp]
        L.oracle_dispatch_bwd.restype = ctypes.c_int
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e4m3_round_array.argtypes = [vp, vp, i64]
        L.oracle_e4m3_round_array.restype = None
        L.oracle_fp8_quantize_row.argtypes = [i64, vp, vp, vp]
        L.oracle_fp8_quantize_row.restype = None
        L.oracle_dispatch_fp8.argtypes = [i64, i64, vp, i64, vp, vp, vp]
        L.oracle_dispatch_fp8.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def bf16_round(values) -> np.ndarray:
    """Round fp32 values to bf16 bit patterns (uint16), nearest-even."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.zeros(v.shape, np.uint16)
    lib().oracle_bf16_round_array(_p(v), _p(out), v.size)
    return out


def capacity_min(T, k, EL, P) -> int:
    return int(lib().oracle_capacity_min(T, k, EL, P))


def check_args(T, k, E, lb, EL, P, sync_free=False, C=0) -> int:
    return int(lib().oracle_check_args(T, k, E, lb, EL, P, int(bool(sync_free)), C))


def check_hidden(H) -> int:
    return int(lib().oracle_check_hidden(H))


@dataclass
class Route:
    rc: int
    map: np.ndarray          # [T,E] uint8
    probs: np.ndarray | None  # [T,E] float32
    tpe: np.ndarray          # [EL] int32
    off: np.ndarray          # [EL+1] int32
    row_of_slot: np.ndarray  # [T,k] int32
    total: int
    flags: int
    R: int
    row_token: np.ndarray    # [R] int32
    row_expert: np.ndarray   # [R] int32
    row_w: np.ndarray | None  # [R] float32
    rows: np.ndarray | None  # [R,H] uint16 (bf16 bits)



def _poison(shape, dtype) -> np.ndarray:
    """An output buffer filled with a pattern the oracle never writes (a NaN
    payload, -7, 0xA5), so that an element it fails to write shows up."""
    dt = np.dtype(dtype)
    fill = {np.dtype(np.uint16): 0x7FC1, np.dtype(np.uint8): 0xA5, np.dtype(np.float32): np.nan,
            np.dtype(np.int32): -7, np.dtype(np.int64): -7}[dt]
    return np.full(shape, fill, dt)


def route(idx, E, lb=0, EL=None, P=1, sync_free=False, C=0, w=None, x=None,
          want_probs=False) -> Route:
    """Routing metadata (and dispatched rows when ``x`` is given).

    idx: [T,k] integer ids (-1 = no expert); w: [T,k] float32 or None;
    x: [T,H] uint16 bf16 bits or None.
    """
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    T, k = idx.shape
    EL = E if EL is None else EL
    w = None if w is None else np.ascontiguousarray(w, dtype=np.float32)
    H = 0
    if x is not None:
        x = np.ascontiguousarray(x, dtype=np.uint16)
        H = x.shape[1]
    Rcap = C if sync_free else T * min(k, max(EL, 1)) + max(EL, 1) * max(P - 1, 0)
    Rcap = max(Rcap, 0)
    m = _poison((T, E), np.uint8)
    probs = _poison((T, E), np.float32) if (want_probs and w is not None) else None
    tpe = _poison(max(EL, 1), np.int32)
    off = _poison(max(EL, 1) + 1, np.int32)
    ros = _poison((T, k), np.int32)
    rt = _poison(max(Rcap, 1), np.int32)
    re = _poison(max(Rcap, 1), np.int32)
    rw = _poison(max(Rcap, 1), np.float32) if w is not None else None
    rows = _poison((max(Rcap, 1), max(H, 1)), np.uint16) if x is not None else None
    total = ctypes.c_int64(0)
    flags = ctypes.c_int32(0)
    rc = lib().oracle_route(T, k, E, lb, EL, P, int(bool(sync_free)), C,
                            _p(idx), _p(w), _p(x), H,
                            _p(m), _p(probs), _p(tpe), _p(off), _p(ros), Rcap,
                            _p(rt), _p(re), _p(rw), _p(rows),
                            ctypes.byref(total), ctypes.byref(flags))
    tot = int(total.value)
    R = C if sync_free else tot
    return Route(rc=rc, map=m, probs=probs, tpe=tpe[:EL], off=off[:EL + 1], row_of_slot=ros,
                 total=tot, flags=int(flags.value), R=R, row_token=rt[:R], row_expert=re[:R],
                 row_w=None if rw is None else rw[:R],
                 rows=None if rows is None else rows[:R, :H])


def combine(idx, row_of_slot, Y, E, lb=0, EL=None, out="bf16"):
    """Per-token fp32 sum of Y rows over primary local slots (ascending slot).
    Y: [R,H] uint16 bf16 bits.  Returns uint16 bf16 bits or float32."""
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    ros = np.ascontiguousarray(row_of_slot, dtype=np.int32)
    Y = np.ascontiguousarray(Y, dtype=np.uint16)
    T, k = idx.shape
    R, H = Y.shape
    EL = E if EL is None else EL
    ob = _poison((T, H), np.uint16) if out == "bf16" else None
    of = _poison((T, H), np.float32) if out == "f32" else None
    rc = lib().oracle_combine(T, k, E, lb, EL, _p(idx), _p(ros), R, H, _p(Y), _p(ob), _p(of))
    if rc != OK:
        raise ValueError(f"oracle_combine rc={rc}")
    return ob if out == "bf16" else of


def combine_bwd(idx, row_of_slot, row_token, grad_out, E, lb=0, EL=None, F=None, R=None):
    """Cached dispatch of grad_out along the rows, plus dw [T,k] when F is given."""
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    ros = np.ascontiguousarray(row_of_slot, dtype=np.int32)
    rt = np.ascontiguousarray(row_token, dtype=np.int32)
    g = np.ascontiguousarray(grad_out, dtype=np.uint16)
    T, k = idx.shape
    H = g.shape[1]
    R = rt.shape[0] if R is None else R
    EL = E if EL is None else EL
    Fa = None if F is None else np.ascontiguousarray(F, dtype=np.uint16)
    gr = _poison((max(R, 1), H), np.uint16)
    dw = _poison((T, k), np.float32) if F is not None else None
    rc = lib().oracle_combine_bwd(T, k, E, lb, EL, _p(idx), _p(ros), _p(rt), R, H, _p(g),
                                  _p(Fa), _p(gr), _p(dw))
    if rc != OK:
        raise ValueError(f"oracle_combine_bwd rc={rc}")
    return gr[:R], dw


def dispatch_bwd(idx, row_of_slot, grad_rows, E, lb=0, EL=None, grad_row_w=None, out="bf16"):
    """Adjoint of dispatch: (grad_x [T,H] bf16 bits or float32, grad_topk_w [T,k] or None)."""
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    ros = np.ascontiguousarray(row_of_slot, dtype=np.int32)
    G = np.ascontiguousarray(grad_rows, dtype=np.uint16)
    T, k = idx.shape
    R, H = G.shape
    EL = E if EL is None else EL
    gw = None if grad_row_w is None else np.ascontiguousarray(grad_row_w, dtype=np.float32)
    ob = _poison((T, H), np.uint16) if out == "bf16" else None
    of = _poison((T, H), np.float32) if out == "f32" else None
    gtw = _poison((T, k), np.float32) if gw is not None else None
    rc = lib().oracle_dispatch_bwd(T, k, E, lb, EL, _p(idx), _p(ros), R, H, _p(G), _p(gw), _p(ob),
                                   _p(of), _p(gtw))
    if rc != OK:
        raise ValueError(f"oracle_dispatch_bwd rc={rc}")
    return (ob if out == "bf16" else of), gtw


# ---------------------------------------------------------------------------
# FP8 dispatch (readings R14..R17 in moe_oracle.c)
# ---------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    """Value of one OCP E4M3 code (NaN for S.1111.111)."""
    return float(lib().oracle_e4m3_value(int(code) & 0xFF))


def e4m3_round(values) -> np.ndarray:
    """fp32 values -> nearest E4M3 codes (uint8), ties to even, magnitude capped at 448."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = _poison(v.shape, np.uint8)
    lib().oracle_e4m3_round_array(_p(v), _p(out), v.size)
    return out


def fp8_quantize(x) -> tuple[np.ndarray, np.ndarray]:
    """Token rows [n,H] (bf16 bits) -> (codes [n,H] uint8, scales [n,H/128] float32)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    n, H = x.shape
    q = _poison((n, H), np.uint8)
    s = _poison((n, H // 128), np.float32)
    for i in range(n):
        lib().oracle_fp8_quantize_row(H, _p(x[i]), _p(q[i]), _p(s[i]))
    return q, s


def dispatch_fp8(x, row_token) -> tuple[np.ndarray, np.ndarray]:
    """FP8 rows [R,H] uint8 and scales [R,H/128] for the rows of a routing."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    rt = np.ascontiguousarray(row_token, dtype=np.int32)
    T, H = x.shape
    R = rt.shape[0]
    q = _poison((max(R, 1), H), np.uint8)
    s = _poison((max(R, 1), H // 128), np.float32)
    rc = lib().oracle_dispatch_fp8(T, H, _p(x), R, _p(rt), _p(q), _p(s))
    if rc != OK:
        raise ValueError(f"oracle_dispatch_fp8 rc={rc}")
    return q[:R], s[:R]
