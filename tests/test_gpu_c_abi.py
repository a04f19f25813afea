"""The activation's C ABI used from plain C: tests/c_abi/swiglu_c_check.c (built by the
package build step) runs forward and backward on a stream, captures them in a HIP graph
and replays it, and checks every output against the CPU oracle's C functions."""
import os
import subprocess

import pytest

from parity import say

pytestmark = pytest.mark.gpu
BINARY = os.path.join(os.path.dirname(__file__), "c_abi", "swiglu_c_check")


def test_c_program_against_oracle():
    assert os.path.exists(BINARY), "tests/c_abi/swiglu_c_check is missing: run __graft_entry__.build()"
    say("[c abi] running tests/c_abi/swiglu_c_check")
    res = subprocess.run([BINARY], capture_output=True, text=True, timeout=240)
    say(res.stdout.strip())
    assert res.returncode == 0, f"exit {res.returncode}\n{res.stdout}\n{res.stderr}"
    assert "C ABI check: ok" in res.stdout
