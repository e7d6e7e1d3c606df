"""The C ABI used from C++ without Python (tests/c_abi_check.cpp, built by
__graft_entry__.build() next to the library): every linear entry point on
hipMalloc'd buffers and a HIP stream, checked against the CPU oracle in the
same process, plus the host-side argument checks. Run as a child process."""
import os
import subprocess

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_abi_check")


def test_c_abi_from_cpp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(BIN), "tests/c_abi_check is not built: run __graft_entry__.build()"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "c_abi_check: all passed" in r.stdout, r.stdout[-3000:]
    assert r.stdout.count("codes, scales exact") == 9
