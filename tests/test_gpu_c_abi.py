"""The C ABI driven from a plain host program (tests/c_abi/abi_smoke.cpp, built
by __graft_entry__.build()): hipMalloc'd buffers, one stream, no Python or
torch between the caller and libbllm.so; results checked against closed forms."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_smoke")


def test_c_program_calls_the_abi():
    assert os.path.exists(EXE), f"{EXE} not built: run __graft_entry__.build()"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi smoke ok" in r.stdout
