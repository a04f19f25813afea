"""Sizes past 4 GiB per tensor, hipGraph replay of the MoE ops, and concurrent streams.

The large-tensor test checks sampled rows: the oracle recomputes just those rows
(rows are independent, a property pinned on the oracle), on the same bytes the
kernel read, copied back from the device.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.moe as moe_oracle
from bf16cmp import grad_probs_violations, ulp_distance
from memory_bound_elementwise_amd import (moe_residual_add, moe_squared_relu_probs_bwd,
                                          moe_squared_relu_probs_fwd, moe_unpermute_expert_order,
                                          swiglu_probs_bwd, swiglu_probs_fwd)
from parity import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def test_activation_past_4gib():
    """x of 5.0 GB and grad_x of 5.0 GB: byte offsets beyond 2^32 on every stream."""
    rows, inter = 305_000, 4096
    g = torch.Generator(device=DEV).manual_seed(123)
    say(f"[large] rows={rows} inter={inter}: x {rows * 2 * inter * 2 / 1e9:.1f} GB")
    x = (torch.randn(rows, 2 * inter, device=DEV, generator=g) * 3).to(torch.bfloat16)
    probs = torch.rand(rows, device=DEV, generator=g)
    gy = torch.randn(rows, inter, device=DEV, generator=g).to(torch.bfloat16)
    y = torch.empty(rows, inter, dtype=torch.bfloat16, device=DEV)
    swiglu_probs_fwd(x, probs, y, 7.0)
    del g
    gx = torch.empty_like(x)
    gp = torch.empty_like(probs)
    swiglu_probs_bwd(x, probs, gy, gx, gp, 7.0)
    torch.cuda.synchronize()
    sample = np.unique(np.concatenate([np.arange(0, 4), np.arange(rows - 300, rows),
                                       np.random.default_rng(0).integers(0, rows, 300)]))
    idx = torch.from_numpy(sample).to(DEV)
    xs, gys = _bits(x[idx]), _bits(gy[idx])
    ps = probs[idx].cpu().numpy()
    orc = oracle.get()
    want_y = orc.fwd(xs, ps, 7.0)
    want = orc.bwd(xs, ps, gys, 7.0)
    assert ulp_distance(_bits(y[idx]), want_y).max() <= 1
    assert ulp_distance(_bits(gx[idx]), want["grad_x"]).max() <= 1
    bad = grad_probs_violations(gp[idx].cpu().numpy(), want["grad_probs_f64"], want["row_scale"])
    assert bad.size == 0
    say(f"[large] {sample.size} sampled rows ok")


def test_widest_rows():
    """inter = 2^28, the widest row the C ABI accepts: each row is 131,072 column chunks
    of four vectors per lane, shared by a workgroup's four waves, with chunk offsets up
    to 2^29 bytes. Two rows, every element against the oracle (compared in slices)."""
    rows, inter = 2, 1 << 28
    g = torch.Generator(device=DEV).manual_seed(11)
    say(f"[widest] rows={rows} inter={inter}")
    x = (torch.randn(rows, 2 * inter, device=DEV, generator=g) * 3).to(torch.bfloat16)
    probs = torch.rand(rows, device=DEV, generator=g)
    gy = torch.randn(rows, inter, device=DEV, generator=g).to(torch.bfloat16)
    y = torch.empty(rows, inter, dtype=torch.bfloat16, device=DEV)
    gx = torch.empty_like(x)
    gp = torch.empty_like(probs)
    swiglu_probs_fwd(x, probs, y, 7.0)
    swiglu_probs_bwd(x, probs, gy, gx, gp, 7.0)
    torch.cuda.synchronize()
    xs, gys, ps = _bits(x), _bits(gy), probs.cpu().numpy()
    del x, gy
    say("[widest] kernels done; oracle forward")
    orc = oracle.get()
    want_y = orc.fwd(xs, ps, 7.0)
    got = _bits(y).reshape(-1)
    step = 1 << 24
    for i in range(0, got.size, step):
        assert ulp_distance(got[i:i + step], want_y.reshape(-1)[i:i + step]).max() <= 1, f"y at {i}"
    del want_y, got, y
    say("[widest] y ok; oracle backward")
    want = orc.bwd(xs, ps, gys, 7.0)
    got = _bits(gx).reshape(-1)
    wgx = want["grad_x"].reshape(-1)
    for i in range(0, got.size, step):
        assert ulp_distance(got[i:i + step], wgx[i:i + step]).max() <= 1, f"grad_x at {i}"
    assert grad_probs_violations(gp.cpu().numpy(), want["grad_probs_f64"], want["row_scale"]).size == 0
    say("[widest] ok")


def test_row_counts_past_the_dispatch_limit():
    """70 million rows of 8 columns. One wave per row would take 17.5 million workgroups,
    past the 16,777,215 a dispatch can hold (its work-item count is 32 bits): the default
    grid stops at that many, and the waves of the first 2.9 million rows take a second
    row 67,108,860 rows on. Sampled rows on both sides of that seam, for the activation
    and the soft-clamped squared ReLU, forward and backward, against the oracle."""
    rows, inter = 70_000_000, 8
    seam = 16_777_215 * 4
    sample = np.unique(np.concatenate([np.arange(0, 4), np.arange(seam - 4, seam + 4),
                                       np.arange(rows - 300, rows),
                                       np.random.default_rng(5).integers(0, rows, 300)]))
    idx = torch.from_numpy(sample).to(DEV)
    g = torch.Generator(device=DEV).manual_seed(321)
    say(f"[dispatch limit] activation rows={rows} inter={inter}")
    x = (torch.randn(rows, 2 * inter, device=DEV, generator=g) * 3).to(torch.bfloat16)
    probs = torch.rand(rows, device=DEV, generator=g)
    gy = torch.randn(rows, inter, device=DEV, generator=g).to(torch.bfloat16)
    y = torch.empty(rows, inter, dtype=torch.bfloat16, device=DEV)
    gx = torch.empty_like(x)
    gp = torch.empty_like(probs)
    swiglu_probs_fwd(x, probs, y, 7.0)
    swiglu_probs_bwd(x, probs, gy, gx, gp, 7.0)
    torch.cuda.synchronize()
    xs, gys, ps = _bits(x[idx]), _bits(gy[idx]), probs[idx].cpu().numpy()
    orc = oracle.get()
    assert ulp_distance(_bits(y[idx]), orc.fwd(xs, ps, 7.0)).max() <= 1
    want = orc.bwd(xs, ps, gys, 7.0)
    assert ulp_distance(_bits(gx[idx]), want["grad_x"]).max() <= 1
    assert grad_probs_violations(gp[idx].cpu().numpy(), want["grad_probs_f64"], want["row_scale"]).size == 0
    del x, gx, y

    say(f"[dispatch limit] squared ReLU rows={rows} hidden={inter}")
    xq = (torch.randn(rows, inter, device=DEV, generator=g) * 6).to(torch.bfloat16)
    yq = torch.empty_like(xq)
    gxq = torch.empty_like(xq)
    moe_squared_relu_probs_fwd(xq, probs, yq, clamp_scale=4.0)
    moe_squared_relu_probs_bwd(xq, probs, gy, gxq, gp, clamp_scale=4.0)
    torch.cuda.synchronize()
    mo = moe_oracle.get()
    xqs = _bits(xq[idx])
    assert ulp_distance(_bits(yq[idx]), mo.squared_relu_probs(xqs, ps, clamp_scale=4.0)).max() <= 1
    wq = mo.squared_relu_probs_bwd(xqs, ps, gys, clamp_scale=4.0)
    assert ulp_distance(_bits(gxq[idx]), wq["grad_x"]).max() <= 1
    assert grad_probs_violations(gp[idx].cpu().numpy(), wq["grad_probs_f64"], wq["row_scale"]).size == 0
    say(f"[dispatch limit] {sample.size} sampled rows ok")


def test_moe_ops_graph_replay():
    """One graph holding the squared ReLU forward and backward (device n_used) and the
    unpermute (device valid_tokens); both counts change between replays, with eager work
    in between."""
    rng = np.random.default_rng(3)
    rows, hidden, E = 4096, 1024, 8
    x = torch.from_numpy(rng.standard_normal((rows, hidden)).astype(np.float32) * 3).to(torch.bfloat16).to(DEV)
    p = torch.from_numpy(rng.uniform(0, 1, rows).astype(np.float32)).to(DEV)
    gy = torch.from_numpy(rng.standard_normal((rows, hidden)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    y = torch.empty_like(x)
    gx = torch.empty_like(x)
    gp = torch.empty_like(p)
    n_used = torch.tensor([rows], dtype=torch.int32, device=DEV)
    tokens = 512
    valid = rng.random((tokens, E)) < 0.5
    im = np.full((tokens, E), -1, np.int32)
    r = 0
    for e in range(E):
        ts = np.flatnonzero(valid[:, e])
        im[ts, e] = np.arange(r, r + ts.size)
        r += ts.size
    eo = torch.from_numpy(rng.standard_normal((r, hidden)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    imd = torch.from_numpy(im).to(DEV)
    out = torch.empty(tokens, hidden, device=DEV)
    vt = torch.tensor([tokens], dtype=torch.int32, device=DEV)

    def run():
        moe_squared_relu_probs_fwd(x, p, y, clamp_scale=3.0, n_used=n_used, zero_padding=True)
        moe_squared_relu_probs_bwd(x, p, gy, gx, gp, clamp_scale=3.0, n_used=n_used, zero_padding=True)
        moe_unpermute_expert_order(eo, imd, out, valid_tokens=vt)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    orc = moe_oracle.get()
    xb = _bits(x)
    gyb = _bits(gy)
    eob = _bits(eo)
    for nu, v in ((rows, tokens), (1000, 17), (0, 0), (rows - 1, tokens - 1)):
        n_used.fill_(nu)
        vt.fill_(v)
        y.fill_(float("nan"))
        gx.fill_(float("nan"))
        gp.fill_(-12345.5)
        out.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want_y = orc.squared_relu_probs(xb, p.cpu().numpy(), clamp_scale=3.0, n_used=nu, zero_padding=True)
        assert ulp_distance(_bits(y), want_y).max() <= 1, f"replay n_used={nu}"
        want_b = orc.squared_relu_probs_bwd(xb, p.cpu().numpy(), gyb, clamp_scale=3.0, n_used=nu,
                                            zero_padding=True)
        assert ulp_distance(_bits(gx), want_b["grad_x"]).max() <= 1, f"replay bwd n_used={nu}"
        g = gp.cpu().numpy()
        assert np.all(g[nu:] == -12345.5), f"replay bwd n_used={nu}: slots past n_used written"
        bad = grad_probs_violations(g[:nu], want_b["grad_probs_f64"][:nu], want_b["row_scale"][:nu])
        assert bad.size == 0, f"replay bwd n_used={nu}: grad_probs"
        want_o = orc.unpermute(eob, im, "f32", valid_tokens=v,
                               out=np.full((tokens, hidden), -1.0, np.float32))
        assert np.array_equal(out.cpu().numpy().view(np.uint32), want_o.view(np.uint32)), f"replay valid={v}"
        say(f"[graph] replay n_used={nu} valid_tokens={v} ok")


def test_two_streams_concurrently():
    """The activation backward and the residual add enqueued on two streams at once give
    the same bits as when run alone."""
    g = torch.Generator(device=DEV).manual_seed(5)
    rows, inter = 8192, 2048
    x = (torch.randn(rows, 2 * inter, device=DEV, generator=g) * 3).to(torch.bfloat16)
    probs = torch.rand(rows, device=DEV, generator=g)
    gy = torch.randn(rows, inter, device=DEV, generator=g).to(torch.bfloat16)
    e, sh, res = (torch.randn(4096, 7168, device=DEV, generator=g).to(torch.bfloat16) for _ in range(3))
    gx0, gp0, o0 = torch.empty_like(x), torch.empty_like(probs), torch.empty_like(res)
    swiglu_probs_bwd(x, probs, gy, gx0, gp0, 7.0)
    moe_residual_add(e, sh, res, o0)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        gx, gp, o = torch.empty_like(x), torch.empty_like(probs), torch.empty_like(res)
        with torch.cuda.stream(s1):
            swiglu_probs_bwd(x, probs, gy, gx, gp, 7.0)
        with torch.cuda.stream(s2):
            moe_residual_add(e, sh, res, o)
        outs.append((gx, gp, o))
    torch.cuda.synchronize()
    for gx, gp, o in outs:
        assert torch.equal(gx.view(torch.int16), gx0.view(torch.int16))
        assert torch.equal(gp.view(torch.int32), gp0.view(torch.int32))
        assert torch.equal(o.view(torch.int16), o0.view(torch.int16))
