"""HIP path vs CPU oracle, element by element, on the five seeded workloads and on
reduced copies that span several row rounds with a ragged tail.

All calls go through the C ABI (ctypes binding). Bar: see ``parity.py``.
"""
import numpy as np
import pytest
import torch

from memory_bound_elementwise_amd import swiglu_probs_default_workgroups
from memory_bound_elementwise_amd.workloads import WORKLOADS, make_inputs
from parity import check_parity, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "mid", "headline", "padded", "edge"])
def test_workload_parity_full_size(name):
    """Every output element of the full-size workload, in the launch the bench times."""
    inp = make_inputs(name, seed=0)
    check_parity(inp, label=f"{name} full")


@pytest.mark.parametrize("name,rows", [("mid", 1021), ("edge", 4099), ("padded", 3001),
                                       ("headline", 517), ("tiny", 1)])
def test_workload_parity_reduced(name, rows):
    inp = make_inputs(name, seed=1, rows=rows)
    check_parity(inp, label=f"{name} rows={rows}")


@pytest.mark.parametrize("inter", [8, 16, 24, 64, 512, 520, 1400, 2056, 4096, 8192 + 8])
def test_odd_widths(inter):
    """Widths that leave lanes idle, need several column chunks, or end mid-chunk."""
    from memory_bound_elementwise_amd.workloads import Workload
    w = Workload("odd", rows=333, inter=inter, limit=3.0, x_std=3.0)
    check_parity(make_inputs(w, seed=inter), label=f"inter={inter}")


def test_grid_invariance_and_determinism():
    """Result bits do not depend on the workgroup count or on the run."""
    inp = make_inputs("edge", seed=2, rows=3000)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ref = run_gpu(inp)
    for nwg in (1, 3, cus, 4 * cus, 10 * cus, 0):
        say(f"[grid] workgroups={nwg}")
        got = run_gpu(inp, num_workgroups=nwg)
        for a, b, what in zip(got, ref, ("y", "grad_x", "grad_probs")):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{what} bits changed with {nwg} workgroups"


@pytest.mark.parametrize("inter,n_used,permute,zero_padding", [
    (2048, None, False, False), (2048, 2500, True, True), (4096, 2500, True, False),
    (1536, 2500, True, True), (1408, None, False, False), (2048 + 8, None, False, False)])
def test_default_launch_matches_walks(inter, n_used, permute, zero_padding):
    """The default launch runs straight-line kernels (a row per wave, or a row per
    workgroup cut into four quarters); an explicit workgroup count runs the fixed-grid
    walks. Every output bit, the row sums included, must be the same either way."""
    from memory_bound_elementwise_amd.workloads import Workload
    rows = 3001
    w = Workload("walks", rows=rows, inter=inter, limit=7.0, x_std=3.0, probs="topk_softmax",
                 n_used=n_used, permute=permute, zero_padding=zero_padding)
    inp = make_inputs(w, seed=inter + 7)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ref = run_gpu(inp)
    check_parity(inp, label=f"default launch inter={inter}")
    for nwg in (1, 3, cus, 4 * cus, rows, -(-rows // 4)):
        say(f"[walks] inter={inter} workgroups={nwg}")
        got = run_gpu(inp, num_workgroups=nwg)
        for a, b, what in zip(got, ref, ("y", "grad_x", "grad_probs")):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), \
                f"{what} bits differ between the default launch and {nwg} workgroups"


def test_row_subset_invariance():
    """A row's bits do not depend on the other rows in the launch (batch invariance)."""
    full = make_inputs("mid", seed=3, rows=600)
    ref = run_gpu(full)
    sub = np.arange(100, 357)
    part = dict(full, x=full["x"][sub], probs=full["probs"][sub], grad_y=full["grad_y"][sub])
    got = run_gpu(part)
    assert np.array_equal(got[0], ref[0][sub])
    assert np.array_equal(got[1], ref[1][sub])
    assert np.array_equal(got[2].view(np.uint32), ref[2][sub].view(np.uint32))


@pytest.mark.parametrize("inter", [256, 2048, 4096])
def test_no_grad_probs_pointer(inter):
    """grad_probs = NULL skips the reduction and leaves grad_x unchanged. At 2,048 and
    4,096 columns the default launch is the quarter-row kernel, whose row-sum barrier is
    taken only for live rows with a grad_probs pointer: padding rows, dummy rows and a
    NULL pointer must all go through without it."""
    from memory_bound_elementwise_amd.workloads import Workload
    w = Workload("nogp", rows=700, inter=inter, limit=7.0, x_std=3.0, probs="topk_softmax",
                 n_used=650, permute=True, zero_padding=True)
    inp = make_inputs(w, seed=inter + 4)
    pm = inp["permutation_map"].copy()
    pm[[5, 77, 300]] = -1
    inp["permutation_map"] = pm
    _, gx_ref, _ = run_gpu(inp, do_fwd=False)
    check_parity(inp, label=f"no-grad_probs reference inter={inter}")
    _, gx, gp = run_gpu(inp, do_fwd=False, grad_probs=False)
    assert gp is None and np.array_equal(gx, gx_ref)


@pytest.mark.parametrize("n_used", [0, 1, 29999, 30000, 32768, 40000, -7])
def test_padded_n_used_values(n_used):
    inp = make_inputs("padded", seed=5, rows=4096)
    inp["n_used"] = n_used
    check_parity(inp, label=f"padded n_used={n_used}")


@pytest.mark.parametrize("zero_padding", [False, True])
def test_dummy_map_entries(zero_padding):
    """Map entries outside [0, rows) mark interior dummy rows."""
    inp = make_inputs("padded", seed=6, rows=2048)
    pm = inp["permutation_map"].copy()
    rng = np.random.default_rng(0)
    dummy = rng.choice(2048, size=100, replace=False)
    pm[dummy[:50]] = -1
    pm[dummy[50:]] = 2048 + rng.integers(0, 1000, size=50)
    inp["permutation_map"] = pm
    inp["zero_padding"] = zero_padding
    check_parity(inp, label=f"dummy entries zero_padding={zero_padding}")


@pytest.mark.parametrize("inter", [2048, 4096])
@pytest.mark.parametrize("zero_padding", [False, True])
def test_row_bookkeeping_on_shared_rows(inter, zero_padding):
    """The backward shares these rows among a workgroup's four waves (a barrier per row
    with a slot): device n_used, a permutation with interior dummy entries, and padding
    rows must behave as on whole-row walks."""
    from memory_bound_elementwise_amd.workloads import Workload
    rows = 3001
    w = Workload("shared", rows=rows, inter=inter, limit=7.0, x_std=3.0, probs="topk_softmax",
                 n_used=2500, permute=True, zero_padding=zero_padding)
    inp = make_inputs(w, seed=inter + zero_padding)
    pm = inp["permutation_map"].copy()
    rng = np.random.default_rng(inter)
    dummy = rng.choice(2500, size=60, replace=False)
    pm[dummy[:30]] = -1
    pm[dummy[30:]] = rows + rng.integers(0, 100, size=30)
    inp["permutation_map"] = pm
    for n_used in (2500, 1, 0):
        inp["n_used"] = n_used
        check_parity(inp, label=f"shared rows inter={inter} zp={zero_padding} n_used={n_used}")


def test_default_workgroups():
    """Rows of at most two column chunks: one wave per row. Three chunks: at most one
    workgroup per CU, with no round of rows left mostly idle. Four or more: one workgroup
    per row, its four waves sharing the row's chunks. Never past the dispatch limit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = WORKLOADS["headline"].rows
    # forward: 2048 columns = 2 chunks of 2 (one wave per row), 6144 = 3 chunks, 8192 = 4 chunks
    wg = swiglu_probs_default_workgroups("fwd", rows, WORKLOADS["headline"].inter)
    say(f"[launch] fwd inter {WORKLOADS['headline'].inter}: {wg} workgroups")
    assert wg == -(-rows // 4)
    wg = swiglu_probs_default_workgroups("fwd", rows, 6144)
    waves = wg * 4
    rounds = -(-rows // waves)
    say(f"[launch] fwd inter 6144: {wg} workgroups on {cus} CUs, {rounds} row rounds")
    assert cus // 2 <= wg <= cus and rounds * waves - rows < waves
    assert swiglu_probs_default_workgroups("fwd", rows, 8192) == rows
    # backward: rows of 4 or more vectors per lane are shared by the four waves
    for inter in (2048, 6144, 8192):
        wg = swiglu_probs_default_workgroups("bwd", rows, inter)
        say(f"[launch] bwd inter {inter}: {wg} workgroups")
        assert wg == rows
    assert swiglu_probs_default_workgroups("bwd", rows, 1536) == -(-rows // 4)   # 3 vectors per lane
    # a dispatch holds its work-item count in 32 bits: at most 16,777,215 workgroups of 256
    for direction, r, inter in (("fwd", 67_108_860, 8), ("fwd", 70_000_000, 8), ("bwd", 70_000_000, 8),
                                ("bwd", 16_777_216, 2048), ("fwd", 2_000_000_000, 8192)):
        assert swiglu_probs_default_workgroups(direction, r, inter) == 16_777_215, (direction, r, inter)
    assert swiglu_probs_default_workgroups("fwd", 67_108_859, 8) == 16_777_215
    assert swiglu_probs_default_workgroups("fwd", 67_108_856, 8) == 16_777_214
