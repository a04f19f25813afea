"""Plant one mistake at a time in a copy of the oracle's C source, on the CPU, and
require that at least one pin fails for each. This shows the pins are sensitive
to the plausible slips (a dropped term, a wrong sign, index or operand, an
exclusive mask, a different rounding) rather than only to the code as written.
"""
import os
import shutil
import tempfile

import pytest

import oracle
from oracle import build as obuild
from oracle_pins import ALL_PINS

# (name, text in swiglu_oracle.c, replacement). Each text must occur exactly once.
MUTANTS = [
    ("dropped_one_in_dsilu", "sig * (1.0f + cg * (1.0f - sig))", "sig * (cg * (1.0f - sig))"),
    ("exclusive_gate_mask", "int in_gate = (a <= L);", "int in_gate = (a < L);"),
    ("exclusive_up_mask", "(b >= -L) && (b <= L)", "(b > -L) && (b <= L)"),
    ("lower_clamp_on_gate", "return (a > L) ? L : a;", "return (a > L) ? L : ((a < -L) ? -L : a);"),
    ("wrong_sign_in_exp", "1.0f / (1.0f + expf(-z))", "1.0f / (1.0f + expf(z))"),
    ("fwd_dropped_probs", "yr[j] = oracle_bf16_rne((s * cu) * p);", "yr[j] = oracle_bf16_rne(s * cu);"),
    ("fwd_used_gate_for_up", "float cu = clamp_up(widen(up[j]), A->L);",
     "float cu = clamp_up(widen(gate[j]), A->L);"),
    ("dup_wrong_operand", "float du = in_up ? gp * s : 0.0f;", "float du = in_up ? gp * cg : 0.0f;"),
    ("halves_swapped", "dgate[j] = oracle_bf16_rne(dg);\n            dup[j] = oracle_bf16_rne(du);",
     "dgate[j] = oracle_bf16_rne(du);\n            dup[j] = oracle_bf16_rne(dg);"),
    ("grad_probs_times_p", "float term = g * (s * cu);", "float term = g * (s * cu) * p;"),
    ("round_half_up", "drop > 0x8000u || (drop == 0x8000u && (keep & 1u))", "drop >= 0x8000u"),
    ("truncating_round", "keep += 1u; /* a carry", "keep += 0u; /* a carry"),
    ("probs_not_gathered", "const float p = A->probs[slot];\n        for (int64_t j = 0; j < inter; ++j) {\n            float cg",
     "const float p = A->probs[r];\n        for (int64_t j = 0; j < inter; ++j) {\n            float cg"),
    ("grad_probs_not_scattered", "A->grad_probs[slot] = (float)acc;", "A->grad_probs[r] = (float)acc;"),
    ("n_used_off_by_one", "if (r >= bound)\n        return -1;", "if (r > bound)\n        return -1;"),
    ("dummy_entry_accepted", "if (s < 0 || s >= rows)", "if (s < 0 || s > rows)"),
    ("padding_not_zeroed", "memset(yr, 0, (size_t)inter * sizeof(uint16_t));", "(void)yr;"),
    ("f64_dropped_one", "(sig * (1.0 + cg * (1.0 - sig)))", "(sig * (cg * (1.0 - sig)))"),
    ("f64_wrong_mask", "dup[j] = (b >= -limit && b <= limit)", "dup[j] = (b >= -limit && b < limit)"),
]


def _pins_fail(orc):
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    return failed


@pytest.fixture(scope="module")
def source_text():
    with open(obuild.SOURCE) as fh:
        return fh.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(source_text, name, old, new):
    assert source_text.count(old) == 1, f"mutation site for {name} not unique/found"
    tmp = tempfile.mkdtemp(prefix="oracle_mutant_")
    try:
        src = os.path.join(tmp, "mutant.c")
        with open(src, "w") as fh:
            fh.write(source_text.replace(old, new))
        lib = obuild.compile_oracle(src, os.path.join(tmp, "libmutant.so"))
        failed = _pins_fail(oracle.Oracle(lib))
        assert failed, f"no pin caught the planted mistake {name}"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
