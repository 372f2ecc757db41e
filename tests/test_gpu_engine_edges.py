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


# Rows of very different magnitude in one batch.  The 16-bit engine packs two
# rows into the real and imaginary parts of one complex signal, so without a
# scale of their own a small row would carry rounding errors of the order of
# its partner's values.  Every row must meet the bar relative to its own
# magnitude, and an all-zero row must come out exactly zero.
_MIXED = {"f16": [1.0, 1e-3, 0.0, 1.0, 30.0, 1e-2, 1.0, 0.0, 1e-4],
          "bf16": [1.0, 1e-6, 0.0, 1.0, 1e8, 1e-2, 1e-12, 0.0, 3.0]}


@pytest.mark.parametrize("io", ["f16", "bf16"])
@pytest.mark.parametrize("N", [200, 1024, 4096, 8192])
def test_rows_of_different_magnitude(io, N):
    from parity_util import row_rel_l2
    sc = _MIXED[io]
    B, H = len(sc), 2
    label = "mixed-magnitude rows io=%s B=%d H=%d N=%d" % (io, B, H, N)
    say(label)
    g = wl.gen(31 * N)
    u = (torch.randn(B, H, N, generator=g, dtype=torch.float64) *
         torch.tensor(sc, dtype=torch.float64)[:, None, None]).to(DT[io])
    f = wl.random_env_filter(H, N, g)
    D = wl.normal((H,), g)
    dev = device()
    y = to_np(pkg.fft_conv(u.to(dev), f.to(dev), D.to(dev)))
    ref = oracle.causal_conv(u, f, D)
    rows = row_rel_l2(y.reshape(B * H, N), ref.reshape(B * H, N)).reshape(B, H)
    say("  per-row rel_l2 max by batch row: " + " ".join("%.1e" % r for r in rows.max(axis=1)))
    for b, s in enumerate(sc):
        if s == 0.0:
            assert np.count_nonzero(y[b]) == 0, (label, b)
        else:
            assert rows[b].max() <= TOL[io], (label, b, s, float(rows[b].max()))


@pytest.mark.parametrize("io", ["f16", "bf16"])
def test_state_pass_rows_of_different_magnitude(io):
    """State passing pairs chunk rows of consecutive (batch, chunk) index,
    across batch rows when the chunk count is odd."""
    from parity_util import cplx, row_rel_l2
    sc = [1.0, 1e-3, 0.0]
    B, H, S, T = len(sc), 2, 16, 1024
    N = 3 * T
    label = "state_pass mixed-magnitude rows io=%s B=%d H=%d N=%d T=%d" % (io, B, H, N, T)
    say(label)
    g = wl.gen(4242)
    u = (torch.randn(B, H, N, generator=g, dtype=torch.float64) *
         torch.tensor(sc, dtype=torch.float64)[:, None, None]).to(DT[io])
    p = wl.diag_ssm_params(H, S, g)
    D = wl.normal((H,), g)
    dev = device()
    d = {k: v.to(dev) for k, v in p.items()}
    y = to_np(pkg.state_pass(u.to(dev), d["A"], d["Bm"], d["C"], d["dt"], D.to(dev), T))
    ref = oracle.ssm_recurrence(u, cplx(p["A"]), cplx(p["Bm"]), cplx(p["C"]), to_np(p["dt"]), to_np(D))
    rows = row_rel_l2(y.reshape(B * H, N), ref.reshape(B * H, N)).reshape(B, H)
    say("  per-row rel_l2 max by batch row: " + " ".join("%.1e" % r for r in rows.max(axis=1)))
    for b, s in enumerate(sc):
        if s == 0.0:
            assert np.count_nonzero(y[b]) == 0, (label, b)
        else:
            assert rows[b].max() <= TOL[io], (label, b, s, float(rows[b].max()))


@pytest.mark.parametrize("io", ["f16", "bf16"])
def test_state_pass_extreme_scales(io):
    """16-bit state passing with inputs, initial states and SSM parameters far
    from unit scale: rows whose magnitudes need the per-step power-of-two
    input scale (bf16 beyond fp16's range), an initial state much larger than
    the inputs (the carried state's fp16 scale), small B and large C (the
    channel tables' scales); every row and the final state against the
    recurrence."""
    from parity_util import cplx, row_rel_l2
    big, small, xs = (1e12, 1e-12, 1e10) if io == "bf16" else (1e2, 1e-2, 10.0)
    sc = [big, small, 1.0]
    B, H, S, T = len(sc), 3, 16, 512
    N = 4 * T
    label = "state_pass extreme scales io=%s B=%d H=%d N=%d T=%d" % (io, B, H, N, T)
    say(label)
    g = wl.gen(5151)
    u = (torch.randn(B, H, N, generator=g, dtype=torch.float64) *
         torch.tensor(sc, dtype=torch.float64)[:, None, None]).to(DT[io])
    p = wl.diag_ssm_params(H, S, g)
    p["Bm"] = p["Bm"] * 1e-3
    p["C"] = p["C"] * 20.0
    p["A"][1, :4, 0] = 0.0  # a few neutral modes in one channel
    D = wl.normal((H,), g)
    xi = (torch.randn(B, H, S, dtype=torch.float64, generator=g)
          + 1j * torch.randn(B, H, S, dtype=torch.float64, generator=g)) * xs
    xi = xi.to(torch.complex64)
    dev = device()
    d = {k: v.to(dev) for k, v in p.items()}
    y, x = pkg.state_pass(u.to(dev), d["A"], d["Bm"], d["C"], d["dt"], D.to(dev), T, x_in=xi.to(dev),
                          return_state=True)
    torch.cuda.synchronize()
    y = to_np(y)
    ref, xr = oracle.ssm_recurrence(u, cplx(p["A"]), cplx(p["Bm"]), cplx(p["C"]), to_np(p["dt"]), to_np(D),
                                    x_in=xi.numpy().astype(np.complex128), return_state=True)
    assert np.isfinite(y).all(), label
    rows = row_rel_l2(y.reshape(B * H, N), ref.reshape(B * H, N)).reshape(B, H)
    gx = x.cpu().numpy().astype(np.complex128)
    errx = float(np.linalg.norm(gx - xr) / np.linalg.norm(xr))
    say("  per-row rel_l2 max by batch row: " + " ".join("%.1e" % r for r in rows.max(axis=1))
        + "  state %.1e" % errx)
    assert rows.max() <= TOL[io], (label, float(rows.max()))
    assert errx <= 1e-3, (label, errx)
