"""The streaming probe's kernels on the GPU: what each writes (the mixed streams' XOR,
the write-only fill, the read-only stream's conditional sink store), on lengths that
end inside a 4 KiB block, for the default grid and a small explicit one."""
import pytest
import torch

from memory_bound_elementwise_amd.hbm_probe import hbm_probe_fill, hbm_probe_read, hbm_probe_stream
from parity import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_WORDS = (1 << 20) + 4 * 37          # 16-byte vectors: a ragged last block


def _rand_words(n, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randint(-2 ** 31, 2 ** 31 - 1, (n,), generator=g, dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("ns,nd", [(1, 1), (2, 1), (3, 2), (1, 2), (2, 2), (3, 1)])
@pytest.mark.parametrize("nwg", [0, 7])
def test_stream_xor(ns, nd, nwg):
    say(f"[probe stream] {ns}:{nd} nwg={nwg}")
    srcs = [_rand_words(N_WORDS, 10 + s) for s in range(ns)]
    dsts = [torch.full((N_WORDS,), -1, dtype=torch.int32, device=DEV) for _ in range(nd)]
    hbm_probe_stream(srcs, dsts, num_workgroups=nwg)
    torch.cuda.synchronize()
    want = srcs[0].clone()
    for s in srcs[1:]:
        want ^= s
    for d in dsts:
        assert torch.equal(d, want)


@pytest.mark.parametrize("nd", [1, 2])
@pytest.mark.parametrize("nwg", [0, 7])
def test_fill(nd, nwg):
    say(f"[probe fill] {nd} nwg={nwg}")
    guard = torch.full((N_WORDS + 64,), -1, dtype=torch.int32, device=DEV)
    dsts = [guard[:N_WORDS]] + [torch.full((N_WORDS,), -1, dtype=torch.int32, device=DEV)
                                for _ in range(nd - 1)]
    hbm_probe_fill(dsts, 0x12345678, num_workgroups=nwg)
    torch.cuda.synchronize()
    for d in dsts:
        assert bool((d == 0x12345678).all())
    assert bool((guard[N_WORDS:] == -1).all()), "fill wrote past the end"


@pytest.mark.parametrize("ns", [1, 2, 3])
@pytest.mark.parametrize("nwg", [0, 7])
def test_read_only_sink(ns, nwg):
    """Sources of one repeated word: an impossible key leaves the sink alone; the key
    every lane's XOR equals makes the lanes store it (so the loads took place)."""
    say(f"[probe read] {ns} nwg={nwg}")
    w = 0x3F803F80
    srcs = [torch.full((N_WORDS,), w, dtype=torch.int32, device=DEV) for _ in range(ns)]
    sink = torch.full((8,), -1, dtype=torch.int32, device=DEV)
    hbm_probe_read(srcs, 0x0BADF00D, sink, num_workgroups=nwg)
    torch.cuda.synchronize()
    assert bool((sink == -1).all())
    # with the default grid every lane reads a whole number of 4-vector blocks; with an
    # explicit grid a lane's count varies, so only the all-zero case is grid-independent
    zeros = [torch.zeros(N_WORDS, dtype=torch.int32, device=DEV) for _ in range(ns)]
    hbm_probe_read(zeros, 0, sink, num_workgroups=nwg)
    torch.cuda.synchronize()
    assert bool((sink[:4] == 0).all()) and bool((sink[4:] == -1).all())
