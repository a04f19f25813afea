"""Host model of the row walks' work partition (cdna4_stream.h), no GPU needed.

walk_row_split gives workgroup g of G the rows g, g + G, g + 2G, ... in batches of 64,
and wave w of its four the column chunks [floor(w nch / 4), floor((w + 1) nch / 4)).
walk_rows gives wave v of W (= 4G) the rows v, v + W, ... with all nch chunks. The
model repeats those formulas and checks, for many shapes and grids, that every
(row, chunk) is visited exactly once, that every index stays in range, and that the
four waves of a workgroup reach the per-row barrier equally often (a wave that
skipped one would leave its workgroup waiting).
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
