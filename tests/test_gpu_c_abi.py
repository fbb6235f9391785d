"""The library called from a plain C program (tests/c_api/abi_check.c): no
Python, no torch, only the header, the shared library and the HIP runtime.
The program runs a top-1 layer in both modes and checks the identity
combine(dispatch(x)) = x, the counts, offsets, rows of slots, pad and
sentinel rows, the dispatch backward and an error path; it prints "abi ok"."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_api", "abi_check")


def test_c_program_drives_the_library():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built: run __graft_entry__.build()")
    print("[c abi] running " + EXE, flush=True)
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(res.stdout, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "abi ok" in res.stdout
