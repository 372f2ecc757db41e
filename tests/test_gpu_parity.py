"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Every case prints its name and shape before touching the GPU.  Inputs come
from the seeded generators in fft_long_convolution_flashconv_amd.workloads;
the oracle sees exactly the rounded values the GPU sees.  Bars: relative L2
<= 1e-5 for fp32 I/O and <= 2e-2 for fp16/bf16 I/O (fp32 accumulation); the
convolution term alone (D*u removed from both sides) must meet the same bar.
"""
import numpy as np
import pytest
import torch

import fft_long_convolution_flashconv_amd as pkg
from fft_long_convolution_flashconv_amd import workloads as wl
import oracle
from parity_util import TOL, cplx, device, rel_l2, row_rel_l2, say, to_np

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _conv_inputs(B, H, N, io, seed):
    g = wl.gen(seed)
    u = wl.normal((B, H, N), g, dtype=DT[io])
    f = wl.random_env_filter(H, N, g)
    D = wl.normal((H,), g)
    return u, f, D


def _check_conv(u, f, D, y, io, label):
    ref = oracle.causal_conv(u, f, D)
    got = to_np(y)
    err = rel_l2(got, ref)
    du = to_np(D)[None, :, None] * to_np(u)
    err_conv = rel_l2(got - du, ref - du)
    say("  %s rel_l2=%.3e conv_only=%.3e" % (label, err, err_conv))
    assert err <= TOL[io], (label, err)
    # The convolution term alone: D*u is removed from both sides.  For bf16
    # output the rounding of y (dominated by D*u) already reaches ~1e-2 of a
    # small convolution term, so that case is reported, not asserted.
    if io != "bf16":
        assert err_conv <= TOL[io] * (10 if io == "f32" else 1), (label, err_conv)


# ------------------------------------------------------------------ fft_conv

@pytest.mark.parametrize("io", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("N", [1, 5, 16, 33, 100, 256, 1000, 1024, 3000])
def test_fft_conv_shapes(io, N):
    dev = device()
    for B in (1, 3):
        H = 3
        label = "fft_conv io=%s B=%d H=%d N=%d" % (io, B, H, N)
        say(label)
        u, f, D = _conv_inputs(B, H, N, io, seed=N * 7 + B)
        y = pkg.fft_conv(u.to(dev), f.to(dev), D.to(dev))
        torch.cuda.synchronize()
        _check_conv(u, f, D, y, io, label)


@pytest.mark.parametrize("io", ["f16", "bf16"])
@pytest.mark.parametrize("N", [200, 256, 500, 1000, 2000])
def test_fft_conv_batch_sizes(io, N):
    """Batches on both sides of half a round of signals (the 16-bit engine
    takes a half-width workgroup shape for batches that fill at most half a
    round at 2N <= 4096), each with every row checked."""
    dev = device()
    H = 3
    for B in (1, 2, 3, 4, 5, 8, 9, 16, 17):
        label = "fft_conv io=%s B=%d H=%d N=%d" % (io, B, H, N)
        say(label)
        u, f, D = _conv_inputs(B, H, N, io, seed=N * 13 + B)
        y = pkg.fft_conv(u.to(dev), f.to(dev), D.to(dev))
        torch.cuda.synchronize()
        got, ref = to_np(y), oracle.causal_conv(u, f, D)
        rows = row_rel_l2(got.reshape(-1, N), ref.reshape(-1, N))
        assert rows.max() <= TOL[io], (label, rows.max())


@pytest.mark.parametrize("io", ["f32", "f16"])
@pytest.mark.parametrize("N", [4096, 8192])
def test_fft_conv_long_block(io, N):
    dev = device()
    B, H = 2, 2
    label = "fft_conv io=%s B=%d H=%d N=%d" % (io, B, H, N)
    say(label)
    u, f, D = _conv_inputs(B, H, N, io, seed=N)
    y = pkg.fft_conv(u.to(dev), f.to(dev), D.to(dev))
    torch.cuda.synchronize()
    _check_conv(u, f, D, y, io, label)


def test_fft_conv_delta_and_impulse_identities():
    """f = delta_0 gives (1 + D) u; u = delta_0 gives f + D delta (fp32)."""
    dev = device()
    B, H, N = 2, 4, 512
    say("fft_conv identities B=%d H=%d N=%d" % (B, H, N))
    g = wl.gen(11)
    u = wl.normal((B, H, N), g)
    D = wl.normal((H,), g)
    f = torch.zeros(H, N); f[:, 0] = 1.0
    y = to_np(pkg.fft_conv(u.to(dev), f.to(dev), D.to(dev)))
    assert rel_l2(y, (1 + to_np(D))[None, :, None] * to_np(u)) < 1e-6
    fr = wl.random_env_filter(H, N, g)
    ui = torch.zeros(1, H, N); ui[..., 0] = 1.0
    y = to_np(pkg.fft_conv(ui.to(dev), fr.to(dev), D.to(dev)))[0]
    ref = to_np(fr).copy(); ref[:, 0] += to_np(D)
    assert rel_l2(y, ref) < 1e-6


def test_fft_conv_deterministic_and_empty():
    dev = device()
    say("fft_conv determinism B=4 H=8 N=2048 f16")
    u, f, D = _conv_inputs(4, 8, 2048, "f16", seed=5)
    u, f, D = u.to(dev), f.to(dev), D.to(dev)
    y1 = pkg.fft_conv(u, f, D)
    y2 = pkg.fft_conv(u, f, D)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    e = pkg.fft_conv(torch.empty(0, 8, 2048, device=dev, dtype=torch.float16), f, D)
    assert e.shape == (0, 8, 2048)


def test_conv_small_workload():
    w = wl.WORKLOADS["conv_small"]
    dev = device()
    say("workload %s" % w.name)
    inp = wl.make_inputs(w)
    y = pkg.fft_conv(inp["u"].to(dev), inp["f"].to(dev), inp["D"].to(dev))
    torch.cuda.synchronize()
    _check_conv(inp["u"], inp["f"], inp["D"], y, w.dtype, w.name)


# ------------------------------------------------------------------ ssm_filter

@pytest.mark.parametrize("S,N", [(1, 64), (5, 1000), (64, 1024), (64, 8192), (17, 20000)])
def test_ssm_filter(S, N):
    dev = device()
    H = 6
    say("ssm_filter H=%d S=%d N=%d" % (H, S, N))
    p = wl.diag_ssm_params(H, S, wl.gen(S + N))
    f = pkg.ssm_filter(p["A"].to(dev), p["Bm"].to(dev), p["C"].to(dev), p["dt"].to(dev), N)
    ref = oracle.ssm_filter(cplx(p["A"]), cplx(p["Bm"]), cplx(p["C"]), to_np(p["dt"]), N)
    err = rel_l2(to_np(f), ref)
    say("  rel_l2=%.3e" % err)
    assert err <= 1e-5


@pytest.mark.parametrize("io", ["f16", "bf16"])
def test_fft_conv_batch_past_32bit_offsets(io):
    """A batch whose rows span more than 4 GiB: the launcher splits it into
    slices whose row offsets fit 32 bits (checked on rows either side of the
    split and at the ends, odd batch)."""
    dev = device()
    B, H, N = 4099, 64, 8192
    say("fft_conv io=%s B=%d H=%d N=%d (%.1f GiB per activation tensor)" % (io, B, H, N, B * H * N * 2 / 2**30))
    gen = torch.Generator(device=dev).manual_seed(4099)
    u = torch.randn((B, H, N), generator=gen, device=dev, dtype=DT[io])
    g = wl.gen(4099)
    f = wl.random_env_filter(H, N, g)
    D = wl.normal((H,), g)
    y = pkg.fft_conv(u, f.to(dev), D.to(dev))
    torch.cuda.synchronize()
    bs = torch.tensor([0, 1, 2044, 2045, 4089, 4090, 4091, 4097, 4098])
    hs = torch.tensor([0, 63, 17, 40, 5, 31, 62, 1, 33])
    u_s = u[bs.to(dev), hs.to(dev)].cpu()[None]
    ref = oracle.causal_conv(to_np(u_s), to_np(f[hs]), to_np(D[hs]))[0]
    got = to_np(y[bs.to(dev), hs.to(dev)])
    del u, y
    err = rel_l2(got, ref)
    per_row = max(rel_l2(got[i], ref[i]) for i in range(len(bs)))
    say("  rel_l2=%.3e max_row=%.3e" % (err, per_row))
    assert err <= TOL[io] and per_row <= TOL[io]


# ------------------------------------------------------------------ state passing

def _sp_inputs(B, H, N, S, io, seed):
    g = wl.gen(seed)
    u = wl.normal((B, H, N), g, dtype=DT[io])
    p = wl.diag_ssm_params(H, S, g)
    D = wl.normal((H,), g)
    return u, p, D


def _sp_ref(u, p, D, x_in=None):
    return oracle.ssm_recurrence(to_np(u), cplx(p["A"]), cplx(p["Bm"]), cplx(p["C"]), to_np(p["dt"]),
                                 to_np(D), x_in=x_in, return_state=True)


@pytest.mark.parametrize("io", ["f32", "f16", "bf16"])
def test_state_pass_small(io):
    dev = device()
    B, H, N, S, T = 3, 2, 2048, 16, 256
    say("state_pass io=%s B=%d H=%d N=%d S=%d T=%d" % (io, B, H, N, S, T))
    u, p, D = _sp_inputs(B, H, N, S, io, seed=21)
    d = {k: v.to(dev) for k, v in p.items()}
    y, x = pkg.state_pass(u.to(dev), d["A"], d["Bm"], d["C"], d["dt"], D.to(dev), T, return_state=True)
    torch.cuda.synchronize()
    ref, xr = _sp_ref(u, p, D)
    err, errx = rel_l2(to_np(y), ref), rel_l2(x.cpu().numpy().astype(np.complex128), xr)
    say("  rel_l2=%.3e state=%.3e" % (err, errx))
    assert err <= TOL[io]
    assert errx <= (1e-5 if io == "f32" else 1e-3)


def test_state_pass_chunk_invariance_and_split():
    """Every chunk length gives the full-length SSM; two calls joined by the
    state equal one call (the pages: state passing is exact)."""
    dev = device()
    B, H, N, S = 2, 3, 4096, 64
    say("state_pass chunk invariance B=%d H=%d N=%d S=%d" % (B, H, N, S))
    u, p, D = _sp_inputs(B, H, N, S, "f32", seed=33)
    d = {k: v.to(dev) for k, v in p.items()}
    ud, Dd = u.to(dev), D.to(dev)
    ref, xr = _sp_ref(u, p, D)
    for T in (64, 128, 512, 1024, 4096):
        y, x = pkg.state_pass(ud, d["A"], d["Bm"], d["C"], d["dt"], Dd, T, return_state=True)
        err = rel_l2(to_np(y), ref)
        errx = rel_l2(x.cpu().numpy().astype(np.complex128), xr)
        say("  T=%d rel_l2=%.3e state=%.3e" % (T, err, errx))
        assert err <= 1e-5 and errx <= 1e-5
    M = 1536
    y1, x1 = pkg.state_pass(ud[..., :M].contiguous(), d["A"], d["Bm"], d["C"], d["dt"], Dd, 512,
                            return_state=True)
    y2, x2 = pkg.state_pass(ud[..., M:].contiguous(), d["A"], d["Bm"], d["C"], d["dt"], Dd, 512,
                            x_in=x1, return_state=True)
    err = rel_l2(np.concatenate([to_np(y1), to_np(y2)], axis=-1), ref)
    errx = rel_l2(x2.cpu().numpy().astype(np.complex128), xr)
    say("  split at %d rel_l2=%.3e state=%.3e" % (M, err, errx))
    assert err <= 1e-5 and errx <= 1e-5


@pytest.mark.parametrize("io", ["f16", "bf16"])
@pytest.mark.parametrize("T,S", [(64, 16), (256, 64), (1024, 7), (2048, 64), (4096, 64), (8192, 33)])
def test_state_pass_16bit_chunks_and_split(io, T, S):
    """16-bit activations (matrix-core projections): every chunk length from
    one 64-sample block to several column tiles, odd batch, partial mode
    count, and two calls joined by the carried state."""
    dev = device()
    B, H, N = 3, 2, 4 * T
    say("state_pass 16-bit io=%s B=%d H=%d N=%d S=%d T=%d" % (io, B, H, N, S, T))
    u, p, D = _sp_inputs(B, H, N, S, io, seed=T + S)
    d = {k: v.to(dev) for k, v in p.items()}
    ud, Dd = u.to(dev), D.to(dev)
    y, x = pkg.state_pass(ud, d["A"], d["Bm"], d["C"], d["dt"], Dd, T, return_state=True)
    torch.cuda.synchronize()
    ref, xr = _sp_ref(u, p, D)
    err, errx = rel_l2(to_np(y), ref), rel_l2(x.cpu().numpy().astype(np.complex128), xr)
    du = to_np(D)[None, :, None] * to_np(u)
    err_conv = rel_l2(to_np(y) - du, ref - du)
    say("  rel_l2=%.3e conv_only=%.3e state=%.3e" % (err, err_conv, errx))
    assert err <= TOL[io] and err_conv <= TOL[io] and errx <= 1e-3
    M = 3 * T
    y1, x1 = pkg.state_pass(ud[..., :M].contiguous(), d["A"], d["Bm"], d["C"], d["dt"], Dd, T,
                            return_state=True)
    y2, x2 = pkg.state_pass(ud[..., M:].contiguous(), d["A"], d["Bm"], d["C"], d["dt"], Dd, T,
                            x_in=x1, return_state=True)
    err = rel_l2(np.concatenate([to_np(y1), to_np(y2)], axis=-1), ref)
    errx = rel_l2(x2.cpu().numpy().astype(np.complex128), xr)
    say("  split at %d rel_l2=%.3e state=%.3e" % (M, err, errx))
    assert err <= TOL[io] and errx <= 1e-3


@pytest.mark.parametrize("io", ["f16", "bf16"])
@pytest.mark.parametrize("N,T,S", [(4416, 64, 64), (6144, 2048, 20), (64, 64, 1)])
def test_state_pass_16bit_ragged_steps(io, N, T, S):
    """16-bit state passing over lengths that end inside a step of 64 blocks
    (a wave with only part of its 16 blocks, waves with none), from a given
    state: every row against the recurrence, and the final state."""
    dev = device()
    B, H = 3, 2
    say("state_pass ragged io=%s B=%d H=%d N=%d S=%d T=%d" % (io, B, H, N, S, T))
    u, p, D = _sp_inputs(B, H, N, S, io, seed=N + S)
    d = {k: v.to(dev) for k, v in p.items()}
    g = wl.gen(N + S + 1)
    xi = (torch.randn(B, H, S, dtype=torch.float64, generator=g)
          + 1j * torch.randn(B, H, S, dtype=torch.float64, generator=g)).to(torch.complex64)
    y, x = pkg.state_pass(u.to(dev), d["A"], d["Bm"], d["C"], d["dt"], D.to(dev), T, x_in=xi.to(dev),
                          return_state=True)
    torch.cuda.synchronize()
    ref, xr = _sp_ref(u, p, D, x_in=xi.numpy().astype(np.complex128))
    got = to_np(y)
    err, errx = rel_l2(got, ref), rel_l2(x.cpu().numpy().astype(np.complex128), xr)
    rows = row_rel_l2(got.reshape(B * H, N), ref.reshape(B * H, N))
    say("  rel_l2=%.3e max_row=%.3e state=%.3e" % (err, rows.max(), errx))
    assert err <= TOL[io] and rows.max() <= TOL[io] and errx <= 1e-3


@pytest.mark.parametrize("io", ["f16", "bf16"])
def test_state_pass_16bit_same_for_every_chunk_length(io):
    """16-bit state passing carries the state at every 64-sample block, a
    refinement of every chunk grid T: outputs and final states are bitwise
    the same for every valid T."""
    dev = device()
    B, H, N, S = 2, 3, 8192, 64
    say("state_pass T-independence io=%s B=%d H=%d N=%d S=%d" % (io, B, H, N, S))
    u, p, D = _sp_inputs(B, H, N, S, io, seed=808)
    d = {k: v.to(dev) for k, v in p.items()}
    ud, Dd = u.to(dev), D.to(dev)
    y0, x0 = pkg.state_pass(ud, d["A"], d["Bm"], d["C"], d["dt"], Dd, 64, return_state=True)
    for T in (128, 1024, 8192):
        y, x = pkg.state_pass(ud, d["A"], d["Bm"], d["C"], d["dt"], Dd, T, return_state=True)
        torch.cuda.synchronize()
        assert torch.equal(y, y0) and torch.equal(x, x0), T


@pytest.mark.parametrize("io", ["f16", "bf16"])
def test_state_pass_zero_state_equals_none(io):
    """An all-zero x_in gives exactly the result of no x_in (the carried
    state starts at zero either way)."""
    dev = device()
    B, H, N, S, T = 2, 3, 2048, 64, 512
    say("state_pass zero x_in io=%s B=%d H=%d N=%d S=%d T=%d" % (io, B, H, N, S, T))
    u, p, D = _sp_inputs(B, H, N, S, io, seed=77)
    d = {k: v.to(dev) for k, v in p.items()}
    ud, Dd = u.to(dev), D.to(dev)
    y0, x0 = pkg.state_pass(ud, d["A"], d["Bm"], d["C"], d["dt"], Dd, T, return_state=True)
    xz = torch.zeros(B, H, S, dtype=torch.complex64, device=dev)
    y1, x1 = pkg.state_pass(ud, d["A"], d["Bm"], d["C"], d["dt"], Dd, T, x_in=xz, return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(x0, x1)


@pytest.mark.parametrize("io", ["f16", "bf16"])
def test_state_pass_neutral_modes(io):
    """Modes on the unit circle (Re A = 0, |exp(dt A)| = 1, the edge of what
    16-bit state passing supports): the powers of Abar stay in fp16 range and
    the result is the full-length recurrence."""
    dev = device()
    B, H, N, S, T = 2, 3, 4096, 16, 1024
    say("state_pass neutral modes io=%s B=%d H=%d N=%d S=%d T=%d" % (io, B, H, N, S, T))
    u, p, D = _sp_inputs(B, H, N, S, io, seed=505)
    p["A"][..., 0] = 0.0
    d = {k: v.to(dev) for k, v in p.items()}
    y, x = pkg.state_pass(u.to(dev), d["A"], d["Bm"], d["C"], d["dt"], D.to(dev), T, return_state=True)
    torch.cuda.synchronize()
    ref, xr = _sp_ref(u, p, D)
    err, errx = rel_l2(to_np(y), ref), rel_l2(x.cpu().numpy().astype(np.complex128), xr)
    say("  rel_l2=%.3e state=%.3e" % (err, errx))
    assert np.isfinite(to_np(y)).all()
    assert err <= TOL[io] and errx <= 1e-3


def test_state_pass_zero_length_writes_state():
    """No samples: x_out is x_in (or zero without x_in)."""
    dev = device()
    B, H, S = 2, 3, 8
    say("state_pass N=0 B=%d H=%d S=%d" % (B, H, S))
    u, p, D = _sp_inputs(B, H, 0, S, "f16", seed=9)
    d = {k: v.to(dev) for k, v in p.items()}
    xi = torch.randn(B, H, S, dtype=torch.complex64, device=dev)
    y, x = pkg.state_pass(u.to(dev), d["A"], d["Bm"], d["C"], d["dt"], D.to(dev), 64, x_in=xi,
                          return_state=True)
    torch.cuda.synchronize()
    assert y.shape == (B, H, 0) and torch.equal(x, xi)
    y, x = pkg.state_pass(u.to(dev), d["A"], d["Bm"], d["C"], d["dt"], D.to(dev), 64, return_state=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(torch.view_as_real(x)) == 0


# ------------------------------------------------------------------ H3 mix

@pytest.mark.parametrize("io", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("L", [1, 2, 4])
def test_h3_mix_small(io, L):
    dev = device()
    B, N, Dm = 3, 700, 9
    say("h3_mix io=%s B=%d N=%d Dm=%d L=%d" % (io, B, N, Dm, L))
    g = wl.gen(L * 100 + len(io))
    q, k, v = (wl.normal((B, N, Dm), g, dtype=DT[io]) for _ in range(3))
    w = wl.normal((Dm, L), g, std=0.5)
    f = wl.random_env_filter(Dm, N, g)
    D = wl.normal((Dm,), g)
    out = pkg.h3_mix(*(t.to(dev) for t in (q, k, v, w, f, D)))
    torch.cuda.synchronize()
    ref = oracle.h3_mix(q, k, v, w, f, D)
    err = rel_l2(to_np(out), ref)
    say("  rel_l2=%.3e" % err)
    assert err <= TOL[io]


@pytest.mark.parametrize("io", ["f16", "bf16"])
def test_h3_mix_vector_ragged_tiles(io):
    # N and d_model multiples of 8 (16-byte gate accesses) but not of the
    # gates' 64-step x 128-channel tiles
    dev = device()
    B, N, Dm, L = 2, 520, 136, 4
    say("h3_mix io=%s B=%d N=%d Dm=%d L=%d" % (io, B, N, Dm, L))
    g = wl.gen(9000 + len(io))
    q, k, v = (wl.normal((B, N, Dm), g, dtype=DT[io]) for _ in range(3))
    w = wl.normal((Dm, L), g, std=0.5)
    f = wl.random_env_filter(Dm, N, g)
    D = wl.normal((Dm,), g)
    out = pkg.h3_mix(*(t.to(dev) for t in (q, k, v, w, f, D)))
    torch.cuda.synchronize()
    ref = oracle.h3_mix(q, k, v, w, f, D)
    err = rel_l2(to_np(out), ref)
    say("  rel_l2=%.3e" % err)
    assert err <= TOL[io]


# ------------------------------------------------------------------ 16K fused block

@pytest.mark.parametrize("io", ["f16", "bf16"])
@pytest.mark.parametrize("N", [8193, 12000, 16384])
def test_fft_conv_16k_fused_block(io, N):
    """Sequences up to 16K in one fused block (2N = 32768 points) with 16-bit
    activations: odd batch (a partial round), ragged N; also the bidirectional
    copies at that size."""
    dev = device()
    B, H = 3, 2
    label = "fft_conv 16K block io=%s B=%d H=%d N=%d" % (io, B, H, N)
    say(label)
    u, f, D = _conv_inputs(B, H, N, io, seed=N + 1)
    y = pkg.fft_conv(u.to(dev), f.to(dev), D.to(dev))
    torch.cuda.synchronize()
    _check_conv(u, f, D, y, io, label)
    g = wl.random_env_filter(H, N, wl.gen(N + 2))
    yb = pkg.fft_conv_bidir(u.to(dev), f.to(dev), g.to(dev), D.to(dev))
    torch.cuda.synchronize()
    err = rel_l2(to_np(yb), oracle.bidir_conv(u, f, g, D))
    say("  bidir rel_l2=%.3e" % err)
    assert err <= TOL[io]
