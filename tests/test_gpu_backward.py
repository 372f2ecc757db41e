"""GPU parity of the backward pass (h3conv_fft_conv_bwd) against the fp64
oracle's plain gradients (du, df, dD): small shapes over every transform
size and dtype, and the three convolution workloads at full size with every
row checked."""
import numpy as np
import pytest
import torch

import fft_long_convolution_flashconv_amd as pkg
from fft_long_convolution_flashconv_amd import workloads as wl
import oracle
from parity_util import TOL, cplx, device, rel_l2, row_rel_l2, say, to_np

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _check(u, f, D, dy, got, io, label, rows=False):
    du, df, dD = (to_np(t) for t in got)
    r_du, r_df, r_dD = oracle.causal_conv_bwd(u, f, D, dy)
    e = (rel_l2(du, r_du), rel_l2(df, r_df), rel_l2(dD, r_dD))
    msg = "  %s du=%.3e df=%.3e dD=%.3e" % (label, *e)
    worst = 0.0
    if rows:
        B, H, N = du.shape
        worst = max(row_rel_l2(du.reshape(B * H, N), r_du.reshape(B * H, N)).max(), row_rel_l2(df, r_df).max())
        msg += " max_row=%.3e" % worst
    say(msg)
    assert np.isfinite(du).all() and np.isfinite(df).all() and np.isfinite(dD).all()
    assert max(e) <= TOL[io], (label, e)
    assert worst <= TOL[io], (label, worst)


@pytest.mark.parametrize("io", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("N", [1, 7, 64, 100, 256, 500, 1000, 2048, 3000, 8192])
def test_fft_conv_bwd_shapes(io, N):
    dev = device()
    for B in (1, 3):
        H = 3
        label = "fft_conv_bwd io=%s B=%d H=%d N=%d" % (io, B, H, N)
        say(label)
        g = wl.gen(N * 11 + B)
        u = wl.normal((B, H, N), g, dtype=DT[io])
        dy = wl.normal((B, H, N), g, dtype=DT[io])
        f = wl.random_env_filter(H, N, g)
        D = wl.normal((H,), g)
        got = pkg.fft_conv_bwd(u.to(dev), f.to(dev), D.to(dev), dy.to(dev))
        torch.cuda.synchronize()
        _check(u, f, D, dy, got, io, label)


@pytest.mark.parametrize("name", ["conv_small", "conv_1k", "conv_8k"])
def test_fft_conv_bwd_workload_every_row(name):
    """The convolution workloads at full size (filters from the SSM
    parameters where the workload has them), dy ~ N(0, 1) in the I/O type;
    every row of du and every channel of df against the oracle, and a second
    run bitwise equal."""
    w = wl.WORKLOADS[name]
    dev = device()
    say("workload %s backward B=%d H=%d N=%d %s: every row" % (name, w.B, w.H, w.N, w.dtype))
    inp = wl.make_inputs(w)
    d = {k: v.to(dev) for k, v in inp.items()}
    f = pkg.ssm_filter(d["A"], d["Bm"], d["C"], d["dt"], w.N) if "A" in d else d["f"]
    dy = wl.normal((w.B, w.H, w.N), wl.gen(1000 + w.seed), dtype=DT[w.dtype])
    dyd = dy.to(dev)
    got = pkg.fft_conv_bwd(d["u"], f, d["D"], dyd)
    again = pkg.fft_conv_bwd(d["u"], f, d["D"], dyd)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(got, again)), "second run differs"
    _check(inp["u"], to_np(f), inp["D"], dy, got, w.dtype, name, rows=True)


def test_fft_conv_bwd_empty_batch():
    """B == 0: no du rows; df and dD are zeros."""
    dev = device()
    H, N = 4, 300
    say("fft_conv_bwd B=0 H=%d N=%d" % (H, N))
    u = torch.empty(0, H, N, dtype=torch.float16, device=dev)
    f = torch.randn(H, N, device=dev)
    D = torch.randn(H, device=dev)
    df = torch.full((H, N), 7.0, device=dev)
    dD = torch.full((H,), 7.0, device=dev)
    du, df, dD = pkg.fft_conv_bwd(u, f, D, u.clone(), df=df, dD=dD)
    torch.cuda.synchronize()
    assert du.shape == (0, H, N)
    assert torch.count_nonzero(df) == 0 and torch.count_nonzero(dD) == 0


@pytest.mark.parametrize("io", ["f16", "bf16"])
@pytest.mark.parametrize("N", [200, 500, 1000, 2000, 3000])
def test_fft_conv_bwd_mixed_row_magnitudes(io, N):
    """Rows of u and dy of very different magnitudes, crossed so that every
    row's correlation is of the same size (each pair's two rows must keep
    their own weight in the summed filter gradient), and a pair whose
    products are far below the others'."""
    dev = device()
    B, H = 6, 3
    label = "fft_conv_bwd mixed magnitudes io=%s B=%d H=%d N=%d" % (io, B, H, N)
    say(label)
    g = wl.gen(7000 + N)
    su = torch.tensor([1e2, 1e-2, 1.0, 1e-3, 1e-2, 1e-2], dtype=torch.float64).view(B, 1, 1)
    sd = torch.tensor([1e-2, 1e2, 1e-3, 1.0, 1e-2, 1e-2], dtype=torch.float64).view(B, 1, 1)
    u = (wl.normal((B, H, N), g) * su).to(DT[io])
    dy = (wl.normal((B, H, N), g) * sd).to(DT[io])
    f = wl.random_env_filter(H, N, g)
    D = wl.normal((H,), g)
    got = pkg.fft_conv_bwd(u.to(dev), f.to(dev), D.to(dev), dy.to(dev))
    torch.cuda.synchronize()
    _check(u, f, D, dy, got, io, label)


@pytest.mark.parametrize("io", ["f16", "bf16"])
@pytest.mark.parametrize("N", [200, 500, 1000, 2000, 4000, 8000])
def test_fft_conv_bwd_batch_sizes(io, N):
    """Batches of one to several pairs of rounds of the 16-bit backward
    kernels (u and dy rounds over the same row pairs, the sum carried from
    pair to pair), odd and even."""
    dev = device()
    H = 2
    for B in (2, 8, 9, 16, 17):
        label = "fft_conv_bwd io=%s B=%d H=%d N=%d" % (io, B, H, N)
        say(label)
        g = wl.gen(9000 + 17 * N + B)
        u = wl.normal((B, H, N), g, dtype=DT[io])
        dy = wl.normal((B, H, N), g, dtype=DT[io])
        f = wl.random_env_filter(H, N, g)
        D = wl.normal((H,), g)
        got = pkg.fft_conv_bwd(u.to(dev), f.to(dev), D.to(dev), dy.to(dev))
        torch.cuda.synchronize()
        _check(u, f, D, dy, got, io, label, rows=True)
