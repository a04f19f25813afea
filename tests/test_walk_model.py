"""Host model of the row walks' work partition (cdna4_stream.h), no GPU needed.

walk_row_split gives workgroup g of G the rows g, g + G, g + 2G, ... in batches of 64,
and wave w of its four the column chunks [floor(w nch / 4), floor((w + 1) nch / 4)).
walk_rows gives wave v of W (= 4G) the rows v, v + W, ... with all nch chunks. The
model repeats those formulas and checks, for many shapes and grids, that every
(row, chunk) is visited exactly once, that every index stays in range, and that the
four waves of a workgroup reach the per-row barrier equally often (a wave that
skipped one would leave its workgroup waiting). It also models the quarter-row
backward's barrier-free row sum: whatever order the four waves arrive in, exactly one
of them sums, with the same bits as the barrier version.
"""
import pytest

WAVES = 4
BATCH = 64


def split_walk(rows, nch, G, live):
    seen = {}
    for wg in range(G):
        barriers = []
        for w in range(WAVES):
            c_lo = w * nch // WAVES
            nc = (w + 1) * nch // WAVES - c_lo
            assert nc >= 1 and 0 <= c_lo and c_lo + nc <= nch
            n_barriers = 0
            base = wg
            while base < rows:
                nk = min((rows - base + G - 1) // G, BATCH)
                for t in range(nk * nc):
                    k, j = divmod(t, nc)
                    r = base + k * G
                    assert 0 <= r < rows
                    key = (r, c_lo + j)
                    assert key not in seen
                    seen[key] = (wg, w)
                    if j == nc - 1 and r < live:       # rows with a slot store a row sum
                        n_barriers += 1
                base += BATCH * G
            barriers.append(n_barriers)
        assert len(set(barriers)) == 1, (wg, barriers)
    assert len(seen) == rows * nch


def row_walk(rows, nch, G):
    W = G * WAVES
    seen = set()
    for v in range(W):
        base = v
        while base < rows:
            nk = min((rows - base + W - 1) // W, BATCH)
            for t in range(nk * nch):
                k, c = divmod(t, nch)
                r = base + k * W
                assert 0 <= r < rows and (r, c) not in seen
                seen.add((r, c))
            base += BATCH * W
    assert len(seen) == rows * nch


@pytest.mark.parametrize("nch", [4, 5, 7, 8, 13])
def test_split_walk_partition(nch):
    for rows in (1, 3, 64, 65, 777, 4097):
        for G in (1, 2, 3, 7, 64, 777, 1024):
            split_walk(rows, nch, G, live=rows)
            split_walk(rows, nch, G, live=rows // 2)


@pytest.mark.parametrize("nch", [1, 2, 3])
def test_row_walk_partition(nch):
    for rows in (1, 63, 64, 65, 1000):
        for G in (1, 2, 16, 250, 256, 300):
            row_walk(rows, nch, G)


# ---------------------------------------------------------------------------
# The quarter-row backward's row sum (row_sum_last in cdna4_stream.h): each wave writes
# its 64 lane partials, then adds one to a counter zeroed before any wave can arrive;
# the wave that reads 3 (the last) adds the partials lane by lane in wave order 0..3 and
# reduces the 64 lanes with the fixed DPP tree. Modelled in fp32 with numpy for every
# order in which the four waves can arrive: exactly one wave sums, and its bits are those
# of row_sum_split (wave 0 after a barrier, same order).
def _wave_sum(v):
    """The DPP tree of wave_sum on 64 fp32 lanes; returns lane 63's total."""
    import numpy as np
    v = v.astype(np.float32).copy()
    lanes = np.arange(64)

    def step(src_idx, mask=None):
        nonlocal v
        add = v[src_idx]
        if mask is not None:
            add = np.where(mask, add, np.float32(0))
        v = (v + add).astype(np.float32)

    step(lanes ^ 1)                                     # quad_perm [1,0,3,2]
    step(lanes ^ 2)                                     # quad_perm [2,3,0,1]
    step((lanes & ~7) | (7 - (lanes & 7)))              # row_half_mirror
    step((lanes & ~15) | (15 - (lanes & 15)))           # row_mirror
    row = lanes // 16
    step(np.where(row > 0, (row - 1) * 16 + 15, 0), np.isin(row, [1, 3]))   # row_bcast:15
    step(np.full(64, 31), np.isin(row, [2, 3]))                              # row_bcast:31
    return v[63]


def _ordered_lane_sum(parts):
    import numpy as np
    t = parts[0].astype(np.float32)
    for w in range(1, WAVES):
        t = (t + parts[w]).astype(np.float32)
    return t


def test_last_arriver_row_sum_matches_barrier_sum():
    import itertools
    import numpy as np
    rng = np.random.default_rng(0)
    for trial in range(20):
        scale = 10.0 ** rng.integers(-3, 4)
        parts = [(rng.standard_normal(64) * scale).astype(np.float32) for _ in range(WAVES)]
        barrier_total = _wave_sum(_ordered_lane_sum(parts))   # row_sum_split: wave 0 sums
        for order in itertools.permutations(range(WAVES)):
            counter, lds, summed = 0, {}, []
            for w in order:                                  # arrival order
                lds[w] = parts[w]                            # partial written before the count
                before, counter = counter, counter + 1
                if before == WAVES - 1:                      # the last to arrive
                    assert set(lds) == set(range(WAVES))     # every partial is there
                    summed.append(_wave_sum(_ordered_lane_sum([lds[i] for i in range(WAVES)])))
            assert len(summed) == 1, order
            assert np.float32(summed[0]).view(np.uint32) == np.float32(barrier_total).view(np.uint32), order


def test_wave_sum_model_is_a_sum():
    """Pin the DPP-tree model itself: on small integers (exact in fp32) it returns the
    plain sum, so a wrong lane pattern in the model would show here."""
    import numpy as np
    v = np.arange(64, dtype=np.float32)
    assert _wave_sum(v) == np.float32(v.sum())
    v = np.ones(64, dtype=np.float32)
    assert _wave_sum(v) == 64.0
