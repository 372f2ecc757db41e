"""h3conv_state_pass_noalloc: state passing with the library's static scratch
array instead of a workspace argument, for callers that cannot allocate.

Checked through the C ABI against h3conv_state_pass (same kernels, a
workspace allocated by the caller): two calls in a row, the second smaller
than the first, each bitwise equal to the workspace entry point's output and
final state (so nothing left in the shared array by the first call reaches
the second).  The refusal of sizes past the array is a host-side check
(tests/test_boundary.py).
"""
import numpy as np
import pytest
import torch

import fft_long_convolution_flashconv_amd as pkg
from fft_long_convolution_flashconv_amd import workloads as wl
from parity_util import device, say

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _inputs(B, H, N, S, io, seed, dev):
    g = wl.gen(seed)
    u = wl.normal((B, H, N), g, dtype=DT[io]).to(dev)
    p = {k: v.to(dev) for k, v in wl.diag_ssm_params(H, S, g).items()}
    D = wl.normal((H,), g).to(dev)
    xi = torch.view_as_real(torch.randn(B, H, S, dtype=torch.complex64, generator=g)).contiguous().to(dev)
    return u, p, D, xi


def _both(B, H, N, S, T, io, seed):
    dev = device()
    say("noalloc io=%s B=%d H=%d N=%d S=%d T=%d" % (io, B, H, N, S, T))
    u, p, D, xi = _inputs(B, H, N, S, io, seed, dev)
    y_ref, x_ref = pkg.state_pass(u, p["A"], p["Bm"], p["C"], p["dt"], D, T, x_in=xi, return_state=True)
    y = torch.empty_like(u)
    x = torch.empty(B, H, S, 2, device=dev)
    pkg.state_pass_noalloc(u, p["A"], p["Bm"], p["C"], p["dt"], D, T, out=y, x_in=xi, x_out=x)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref), "output differs from h3conv_state_pass"
    assert torch.equal(torch.view_as_complex(x), x_ref), "final state differs from h3conv_state_pass"


@pytest.mark.parametrize("io", ["f16", "bf16"])
def test_noalloc_two_calls_16bit(io):
    # the state-passing workload's full size first, then a smaller call
    w = wl.WORKLOADS["state_64k"]
    _both(w.B, w.H, w.N, w.S, w.T, io, seed=3)
    _both(3, 5, 3 * 1024, 16, 1024, io, seed=4)


def test_noalloc_two_calls_fp32():
    _both(2, 64, 4 * 4096, 64, 4096, "f32", seed=5)
    _both(3, 5, 3 * 256, 7, 256, "f32", seed=6)
