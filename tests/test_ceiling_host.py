"""libmoe_ceiling.so on the CPU: it loads, exports every symbol
include/moe_ceiling.h declares, and refuses bad arguments before launching
anything (every call below fails its host checks)."""
import ctypes
import os
import re

from combine_topk_idx_multihot_amd import ceiling as C

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "moe_ceiling.h")
FAKE = 0x100000  # 16-byte aligned, never dereferenced by the checks


def test_exports_every_declared_symbol():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = set(re.findall(r"\b(moe_ceiling_[a-z_]+)\s*\(", src))
    assert names == set(C.EXPORTS)
    L = C.lib()
    for n in names:
        assert hasattr(L, n)


def test_refusals():
    L = C.lib()
    assert L.moe_ceiling_fill(None, 1024, 1, None) == C.ERR_ARG
    assert L.moe_ceiling_fill(FAKE + 4, 1024, 1, None) == C.ERR_ARG       # misaligned
    assert L.moe_ceiling_fill(FAKE, 1000, 1, None) == C.ERR_ARG           # not a multiple of 16
    assert L.moe_ceiling_fill(FAKE, 1024, 3, None) == C.ERR_ARG           # piece size
    assert L.moe_ceiling_fill(FAKE, 0, 1, None) == C.OK                   # nothing to launch
    assert L.moe_ceiling_copy(FAKE, None, 1024, 1, None) == C.ERR_ARG
    assert L.moe_ceiling_copy(FAKE, FAKE, 1024, 8, None) == C.ERR_ARG
    assert L.moe_ceiling_fill(FAKE, ctypes.c_size_t(1 << 50).value, 1, None) == C.ERR_ARG  # grid
    sc = L.moe_ceiling_scatter
    assert sc(FAKE, 10, 8, 100, 300, FAKE, 1, None) == C.ERR_ARG          # H % 256
    assert sc(FAKE, 10, 0, 100, 256, FAKE, 1, None) == C.ERR_ARG          # k
    assert sc(FAKE, 10, 65, 100, 256, FAKE, 1, None) == C.ERR_ARG
    assert sc(None, 10, 8, 100, 256, FAKE, 1, None) == C.ERR_ARG
    assert sc(FAKE, 10, 8, 100, 256, FAKE, 3, None) == C.ERR_ARG          # segment size
    assert sc(FAKE, -1, 8, 100, 256, FAKE, 1, None) == C.ERR_ARG
    assert sc(None, 0, 8, 100, 256, None, 1, None) == C.OK                # no token
    ga = L.moe_ceiling_gather
    assert ga(FAKE, 10, 8, 100, 300, FAKE, FAKE, None, 2, None) == C.ERR_ARG   # H % 256
    assert ga(FAKE, 10, 0, 100, 256, FAKE, FAKE, None, 2, None) == C.ERR_ARG   # k
    assert ga(FAKE, 10, 65, 100, 256, FAKE, FAKE, None, 2, None) == C.ERR_ARG
    assert ga(FAKE, 10, 8, 100, 256, FAKE, FAKE, None, 3, None) == C.ERR_ARG   # segment size
    assert ga(None, 10, 8, 100, 256, FAKE, FAKE, None, 2, None) == C.ERR_ARG
    assert ga(FAKE, 10, 8, 100, 256, FAKE + 4, FAKE, None, 2, None) == C.ERR_ARG  # Y misaligned
    assert ga(FAKE, 10, 8, 100, 256, FAKE, FAKE + 8, None, 2, None) == C.ERR_ARG  # out misaligned
    assert ga(FAKE, 10, 8, 100, 256, FAKE, None, None, 2, None) == C.ERR_ARG   # read only, no sink
    assert ga(FAKE, -1, 8, 100, 256, FAKE, FAKE, None, 2, None) == C.ERR_ARG
    assert ga(None, 0, 8, 100, 256, None, None, None, 2, None) == C.OK          # no token
    assert L.moe_ceiling_xcd_map(None, 4, None) == C.ERR_ARG
    assert L.moe_ceiling_xcd_map(None, 0, None) == C.OK
