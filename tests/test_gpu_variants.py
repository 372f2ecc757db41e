"""GPU parity of the layer variants against the fp64 oracle: bidirectional
copies of the convolution (h3conv_fft_conv_bidir)."""
import numpy as np
import pytest
import torch

import fft_long_convolution_flashconv_amd as pkg
from fft_long_convolution_flashconv_amd import workloads as wl
import oracle
from parity_util import TOL, cplx, device, rel_l2, row_rel_l2, say, to_np

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.mark.parametrize("io", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("N", [1, 5, 100, 256, 1000, 2048, 4097, 8192])
def test_bidir_shapes(io, N):
    dev = device()
    for B in (1, 3):
        H = 3
        label = "fft_conv_bidir io=%s B=%d H=%d N=%d" % (io, B, H, N)
        say(label)
        gen = wl.gen(N * 13 + B)
        u = wl.normal((B, H, N), gen, dtype=DT[io])
        f = wl.random_env_filter(H, N, gen)
        g = wl.random_env_filter(H, N, gen)
        D = wl.normal((H,), gen)
        y = pkg.fft_conv_bidir(u.to(dev), f.to(dev), g.to(dev), D.to(dev))
        torch.cuda.synchronize()
        ref = oracle.bidir_conv(u, f, g, D)
        err = rel_l2(to_np(y), ref)
        say("  rel_l2=%.3e" % err)
        assert np.isfinite(to_np(y)).all() and err <= TOL[io], (label, err)


def test_bidir_reduces_to_causal_and_reversed():
    """g = 0 gives the causal convolution; f = 0 gives the causal convolution
    of the reversed input with g, reversed back (16-bit, matrix-core path)."""
    dev = device()
    B, H, N = 3, 4, 1500
    say("fft_conv_bidir reductions f16 B=%d H=%d N=%d" % (B, H, N))
    gen = wl.gen(77)
    u = wl.normal((B, H, N), gen, dtype=torch.float16)
    f = wl.random_env_filter(H, N, gen)
    D = wl.normal((H,), gen)
    z = torch.zeros(H, N)
    ud, fd, zd, Dd = u.to(dev), f.to(dev), z.to(dev), D.to(dev)
    y = to_np(pkg.fft_conv_bidir(ud, fd, zd, Dd))
    assert rel_l2(y, oracle.causal_conv(u, f, D)) <= TOL["f16"]
    y = to_np(pkg.fft_conv_bidir(ud, zd, fd, Dd))
    rev = oracle.causal_conv(to_np(u)[..., ::-1].copy(), f, D)[..., ::-1]
    assert rel_l2(y, rev) <= TOL["f16"]


def test_bidir_workload_shape_every_row():
    """The bidirectional workload (the H3-125M convolution shape B=8, H=768,
    N=1024, fp16) with both filters from diagonal-SSM parameters (the
    anti-causal copy has its own draw); every row checked, and a second run
    bitwise equal."""
    w = wl.WORKLOADS["bidir_1k"]
    dev = device()
    say("fft_conv_bidir workload %s B=%d H=%d N=%d f16: every row" % (w.name, w.B, w.H, w.N))
    inp = wl.make_inputs(w)
    d = {k: v.to(dev) for k, v in inp.items()}
    f = pkg.ssm_filter(d["A"], d["Bm"], d["C"], d["dt"], w.N)
    g = pkg.ssm_filter(d["gA"], d["gBm"], d["gC"], d["gdt"], w.N)
    y = pkg.fft_conv_bidir(d["u"], f, g, d["D"])
    again = pkg.fft_conv_bidir(d["u"], f, g, d["D"])
    torch.cuda.synchronize()
    assert torch.equal(y, again), "second run differs"
    ref = oracle.bidir_conv(inp["u"], to_np(f), to_np(g), inp["D"])
    got = to_np(y)
    rows = row_rel_l2(got.reshape(-1, w.N), ref.reshape(-1, w.N))
    err = rel_l2(got, ref)
    say("  rel_l2=%.3e max_row=%.3e" % (err, rows.max()))
    assert err <= TOL["f16"] and rows.max() <= TOL["f16"]


# ------------------------------------------------------------------ multi-head H3

def _mh_inputs(B, N, Dm, dh, L, io, seed):
    gen = wl.gen(seed)
    q, k, v = (wl.normal((B, N, Dm), gen, dtype=DT[io]) for _ in range(3))
    w = wl.normal((Dm, L), gen, std=0.5)
    f = wl.random_env_filter(Dm * dh, N, gen)
    D = wl.normal((Dm * dh,), gen)
    return q, k, v, w, f, D


@pytest.mark.parametrize("io", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("dh,Dm", [(1, 9), (2, 6), (4, 40), (8, 48), (16, 32), (32, 64)])
@pytest.mark.parametrize("N", [77, 1000])
def test_h3_mix_mh_shapes(io, dh, Dm, N):
    dev = device()
    B, L = 2, 4
    label = "h3_mix_mh io=%s B=%d N=%d Dm=%d dh=%d L=%d" % (io, B, N, Dm, dh, L)
    say(label)
    q, k, v, w, f, D = _mh_inputs(B, N, Dm, dh, L, io, seed=N + 10 * dh + Dm)
    out = pkg.h3_mix_mh(*(t.to(dev) for t in (q, k, v, w, f, D)), dh)
    torch.cuda.synchronize()
    ref = oracle.h3_mix_mh(q, k, v, w, f, D, dh)
    err = rel_l2(to_np(out), ref)
    say("  rel_l2=%.3e" % err)
    assert np.isfinite(to_np(out)).all() and err <= TOL[io], (label, err)


@pytest.mark.parametrize("io", ["f32", "f16"])
@pytest.mark.parametrize("L", [1, 2, 3])
def test_h3_mix_mh_shift_taps(io, L):
    """Shift filters of 1 to 3 taps (the other tests use 4)."""
    dev = device()
    B, N, Dm, dh = 2, 300, 16, 4
    label = "h3_mix_mh io=%s B=%d N=%d Dm=%d dh=%d L=%d" % (io, B, N, Dm, dh, L)
    say(label)
    q, k, v, w, f, D = _mh_inputs(B, N, Dm, dh, L, io, seed=400 + L)
    out = pkg.h3_mix_mh(*(t.to(dev) for t in (q, k, v, w, f, D)), dh)
    torch.cuda.synchronize()
    ref = oracle.h3_mix_mh(q, k, v, w, f, D, dh)
    err = rel_l2(to_np(out), ref)
    say("  rel_l2=%.3e" % err)
    assert np.isfinite(to_np(out)).all() and err <= TOL[io], (label, err)


def test_h3_mix_mh_head_dim_one_matches_h3_mix():
    dev = device()
    B, N, Dm, L = 2, 600, 136, 4
    say("h3_mix_mh dh=1 vs h3_mix bf16 B=%d N=%d Dm=%d" % (B, N, Dm))
    q, k, v, w, f, D = _mh_inputs(B, N, Dm, 1, L, "bf16", seed=5)
    a = pkg.h3_mix_mh(*(t.to(dev) for t in (q, k, v, w, f, D)), 1)
    b = pkg.h3_mix(*(t.to(dev) for t in (q, k, v, w, f, D)))
    torch.cuda.synchronize()
    ref = oracle.h3_mix(q, k, v, w, f, D)
    assert rel_l2(to_np(a), ref) <= TOL["bf16"] and rel_l2(to_np(b), ref) <= TOL["bf16"]


def test_h3_mix_mh_125m_width():
    """The H3-125M width (768) in heads of dimension 4, fp16, diagonal-SSM
    filters (one per state entry): every (batch, channel) sequence checked."""
    dev = device()
    B, N, Dm, dh, L = 2, 1024, 768, 4, 4
    say("h3_mix_mh 125M width f16 B=%d N=%d Dm=%d dh=%d" % (B, N, Dm, dh))
    gen = wl.gen(2024)
    q, k, v = (wl.normal((B, N, Dm), gen, dtype=torch.float16) for _ in range(3))
    w = wl.normal((Dm, L), gen, std=0.5)
    p = wl.diag_ssm_params(Dm * dh, 64, gen)
    D = wl.normal((Dm * dh,), gen)
    pd = {kk: vv.to(dev) for kk, vv in p.items()}
    f = pkg.ssm_filter(pd["A"], pd["Bm"], pd["C"], pd["dt"], N)
    out = pkg.h3_mix_mh(q.to(dev), k.to(dev), v.to(dev), w.to(dev), f, D.to(dev), dh)
    torch.cuda.synchronize()
    ref = oracle.h3_mix_mh(q, k, v, w, to_np(f), D, dh)
    got = to_np(out)
    rows = row_rel_l2(got.transpose(0, 2, 1).reshape(-1, N), ref.transpose(0, 2, 1).reshape(-1, N))
    err = rel_l2(got, ref)
    say("  rel_l2=%.3e max_row=%.3e" % (err, rows.max()))
    assert err <= TOL["f16"] and rows.max() <= TOL["f16"]
