"""GPU edge cases of the fp16/bf16 block-FFT path: every transform size, odd
batches (partial rounds of signals), ragged lengths, extreme magnitudes and
coherent (worst-case growth) inputs.  Compared with the fp64 oracle."""
import numpy as np
import pytest
import torch

import fft_long_convolution_flashconv_amd as pkg
from fft_long_convolution_flashconv_amd import workloads as wl
import oracle
from parity_util import TOL, device, rel_l2, say, to_np

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _run(u, f, D, io, label):
    dev = device()
    y = pkg.fft_conv(u.to(dev), f.to(dev), D.to(dev))
    torch.cuda.synchronize()
    ref = oracle.causal_conv(u, f, D)
    err = rel_l2(to_np(y), ref)
    say("  %s rel_l2=%.3e" % (label, err))
    assert np.isfinite(to_np(y)).all(), label
    assert err <= TOL[io], (label, err)
    return err


@pytest.mark.parametrize("io", ["f16", "bf16"])
@pytest.mark.parametrize("N", [65, 128, 129, 300, 512, 700, 1500, 2048, 2049, 5000, 8191])
def test_sizes_and_partial_rounds(io, N):
    for B in (1, 8, 9):
        H = 2
        label = "io=%s B=%d H=%d N=%d" % (io, B, H, N)
        say(label)
        g = wl.gen(N + B)
        u = wl.normal((B, H, N), g, dtype=DT[io])
        f = wl.random_env_filter(H, N, g)
        D = wl.normal((H,), g)
        _run(u, f, D, io, label)


@pytest.mark.parametrize("io,uscale,fscale", [
    ("f16", 1e-4, 1.0), ("f16", 1e3, 1.0), ("f16", 1.0, 1e-4), ("f16", 1.0, 1e3),
    ("bf16", 1e-20, 1.0), ("bf16", 1e20, 1.0), ("bf16", 1.0, 1e-12), ("bf16", 1e-6, 1e8)])
def test_extreme_magnitudes(io, uscale, fscale):
    B, H, N = 3, 3, 1024
    label = "io=%s u*%g f*%g B=%d H=%d N=%d" % (io, uscale, fscale, B, H, N)
    say(label)
    g = wl.gen(7)
    u = (torch.randn(B, H, N, generator=g, dtype=torch.float64) * uscale).to(DT[io])
    f = (wl.random_env_filter(H, N, g).double() * fscale).float()
    D = (wl.normal((H,), g).double() * fscale).float()
    _run(u, f, D, io, label)


@pytest.mark.parametrize("N", [256, 2048, 8192])
def test_coherent_worst_case(N):
    """Constant input and constant filter: every transform sum adds in phase."""
    io = "f16"
    B, H = 2, 2
    label = "coherent io=%s B=%d H=%d N=%d" % (io, B, H, N)
    say(label)
    u = torch.full((B, H, N), 60000.0).to(torch.float16) if N == 256 else torch.full((B, H, N), 3.0).to(torch.float16)
    f = torch.full((H, N), 1.0 / N)
    D = torch.zeros(H)
    _run(u, f, D, io, label)
    f = torch.zeros(H, N); f[:, 0] = 1.0
    _run(u, f, D, io, label + " delta")


def test_zero_input_and_zero_filter():
    dev = device()
    B, H, N = 2, 2, 1024
    say("zeros B=%d H=%d N=%d" % (B, H, N))
    u = torch.zeros(B, H, N, dtype=torch.float16, device=dev)
    f = torch.randn(H, N, device=dev)
    D = torch.randn(H, device=dev)
    assert torch.count_nonzero(pkg.fft_conv(u, f, D)) == 0
    u = torch.randn(B, H, N, device=dev).half()
    y = pkg.fft_conv(u, torch.zeros(H, N, device=dev), torch.zeros(H, device=dev))
    assert torch.count_nonzero(y) == 0
