"""The C ABI from a plain C program (tests/c_abi/abi_main.c: HIP runtime
buffers, the library's entry points, the fp64 oracle as the checker), built by
__graft_entry__.build(); this test runs it on the GPU."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_main")


def test_c_program_against_the_oracle():
    assert os.path.exists(BIN), f"{BIN} is missing: run __graft_entry__.build() first"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all cases passed" in r.stdout
