"""The C ABIs used from plain C. tests/c_abi/swiglu_c_check.c (the activation) and
tests/c_abi/moe_c_check.c (the MoE elementwise operations), built by the package build
step, run every operation on a stream, capture the sequence in a HIP graph and replay it,
and check every output against the CPU oracle's C functions."""
import os
import subprocess

import pytest

from parity import say

pytestmark = pytest.mark.gpu
HERE = os.path.join(os.path.dirname(__file__), "c_abi")


@pytest.mark.parametrize("program, banner", [("swiglu_c_check", "C ABI check: ok"),
                                             ("moe_c_check", "MoE C ABI check: ok")])
def test_c_program_against_oracle(program, banner):
    binary = os.path.join(HERE, program)
    assert os.path.exists(binary), f"tests/c_abi/{program} is missing: run __graft_entry__.build()"
    say(f"[c abi] running tests/c_abi/{program}")
    res = subprocess.run([binary], capture_output=True, text=True, timeout=240)
    say(res.stdout.strip())
    assert res.returncode == 0, f"exit {res.returncode}\n{res.stdout}\n{res.stderr}"
    assert banner in res.stdout
