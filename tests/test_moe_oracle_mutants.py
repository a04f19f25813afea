"""Plant one mistake at a time in a copy of the MoE-ops oracle source (on the CPU)
and require that some pin of ``moe_oracle_pins.py`` fails for each."""
import os
import shutil
import tempfile

import pytest

from oracle import build as obuild
from oracle.moe import MoeOracle
from moe_oracle_pins import ALL_PINS

MUTANTS = [
    ("residual_no_inner_rounding",
     "float t = round_to(load_elem(A->expert, i, A->dt) + load_elem(A->shared, i, A->dt), A->dt);",
     "float t = load_elem(A->expert, i, A->dt) + load_elem(A->shared, i, A->dt);"),
    ("residual_wrong_operand",
     "float t = round_to(load_elem(A->expert, i, A->dt) + load_elem(A->shared, i, A->dt), A->dt);",
     "float t = round_to(load_elem(A->expert, i, A->dt) + load_elem(A->residual, i, A->dt), A->dt);"),
    ("f16_ties_away", "    float r = nearbyintf(n);\n    if (r == 2048.0f)", "    float r = roundf(n);\n    if (r == 2048.0f)"),
    ("f16_subnormal_truncated", "float r = nearbyintf(n);   /* default", "float r = truncf(n);   /* default"),
    ("router_fwd_wrong_prob", "load_elem(A->x, t * hidden + h, A->x_dt) * A->probs[t]);",
     "load_elem(A->x, t * hidden + h, A->x_dt) * A->probs[0]);"),
    ("router_grad_x_no_prob", "store_elem(A->grad_x, t * hidden + h, A->x_dt, g * A->probs[t]);",
     "store_elem(A->grad_x, t * hidden + h, A->x_dt, g);"),
    ("router_grad_probs_times_p", "float term = g * load_elem(A->x, t * hidden + h, A->x_dt);",
     "float term = g * load_elem(A->x, t * hidden + h, A->x_dt) * A->probs[t];"),
    ("sqrelu_square_not_rounded", "float sq = bf16_to_f32(f32_to_bf16(a * a));", "float sq = a * a;"),
    ("sqrelu_scale_inverted", "tanhf(v / A->clamp_scale)", "tanhf(v * A->clamp_scale)"),
    ("sqrelu_no_relu", "float a = c < 0.0f ? 0.0f : c;", "float a = c;"),
    ("sqrelu_map_not_gathered", "const float p = A->probs[slot];", "const float p = A->probs[r];"),
    ("sqrelu_bwd_no_factor_two", "((g * prob) * (2.0f * a)) * sech2", "((g * prob) * a) * sech2"),
    ("sqrelu_bwd_sech2_from_fp32_tanh", "float sech2 = (4.0f * e) / ((1.0f + e) * (1.0f + e));",
     "float sech2 = 1.0f - tanhf(z) * tanhf(z);"),
    ("sqrelu_bwd_sech_not_squared", "float sech2 = (4.0f * e) / ((1.0f + e) * (1.0f + e));",
     "float sech2 = (4.0f * e) / (1.0f + e);"),
    ("sqrelu_bwd_mask_includes_zero", "gx = v > 0.0f ? ((g * prob)", "gx = v >= 0.0f ? ((g * prob)"),
    ("sqrelu_bwd_nan_passes_mask", "gx = v > 0.0f ? (g * prob) * (2.0f * a) : 0.0f;",
     "gx = !(v <= 0.0f) ? (g * prob) * (2.0f * a) : 0.0f;"),
    ("sqrelu_bwd_no_relu", "float a = (c < 0.0f) ? 0.0f : c; /* relu; NaN passes */", "float a = c;"),
    ("sqrelu_bwd_grad_probs_times_p", "const float term = g * ypre;", "const float term = g * ypre * prob;"),
    ("sqrelu_bwd_square_not_rounded", "ypre = bf16_to_f32(f32_to_bf16(a * a));", "ypre = a * a;"),
    ("sqrelu_bwd_no_gather", "const float prob = A->probs[slot];", "const float prob = A->probs[r];"),
    ("sqrelu_bwd_padding_not_zeroed", "if (A->zero_padding && A->grad_x)", "if (0 && A->grad_x)"),
    ("unpermute_reversed", "for (int64_t e = 0; e < E; ++e) {", "for (int64_t e = E - 1; e >= 0; --e) {"),
    ("unpermute_bound_off_by_one", "over_rows(bound, threads, &a, unpermute_rows);",
     "over_rows(bound + (bound < tokens), threads, &a, unpermute_rows);"),
    # a thread's row block one row short: results then depend on the thread count
    ("thread_blocks_drop_a_row", "blk[t] = (row_block_t){args, r, r + n, body};",
     "blk[t] = (row_block_t){args, r, r + n - (t > 0 && n > 1), body};"),
]


def _failed(orc):
    out = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, IndexError):
            out.append(pin.__name__)
    return out


@pytest.fixture(scope="module")
def source_text():
    with open(obuild.MOE_SOURCE) as fh:
        return fh.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(source_text, name, old, new):
    assert source_text.count(old) == 1, f"mutation site for {name} not unique/found"
    tmp = tempfile.mkdtemp(prefix="moe_oracle_mutant_")
    try:
        src = os.path.join(tmp, "mutant.c")
        with open(src, "w") as fh:
            fh.write(source_text.replace(old, new))
        lib = obuild.compile_oracle(src, os.path.join(tmp, "libmutant.so"))
        assert _failed(MoeOracle(lib)), f"no pin caught the planted mistake {name}"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
