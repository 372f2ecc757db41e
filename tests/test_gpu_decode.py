"""GPU parity of the recurrent generation step (h3conv_ssm_step) against the
fp64 oracle recurrence (the same step-by-step definition, started from the
given state).  A state-passing prefix continued by decode steps must equal
the full-length recurrence over the whole sequence."""
import numpy as np
import pytest
import torch

import fft_long_convolution_flashconv_amd as pkg
from fft_long_convolution_flashconv_amd import workloads as wl
import oracle
from parity_util import TOL, cplx, device, rel_l2, row_rel_l2, say, to_np

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _params(H, S, seed):
    g = wl.gen(seed)
    p = wl.diag_ssm_params(H, S, g)
    D = wl.normal((H,), g)
    return g, p, D


def _ref(u, p, D, x_in):
    return oracle.ssm_recurrence(to_np(u), cplx(p["A"]), cplx(p["Bm"]), cplx(p["C"]), to_np(p["dt"]),
                                 to_np(D), x_in=x_in, return_state=True)


@pytest.mark.parametrize("io", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("S,K", [(1, 1), (17, 7), (64, 64), (64, 65), (33, 300)])
def test_ssm_step_from_state(io, S, K):
    dev = device()
    B, H = 3, 5
    say("ssm_step io=%s B=%d H=%d S=%d K=%d" % (io, B, H, S, K))
    g, p, D = _params(H, S, 100 * S + K)
    u = wl.normal((B, H, K), g, dtype=DT[io])
    x0 = torch.randn(B, H, S, dtype=torch.complex64, generator=g)
    d = {k: v.to(dev) for k, v in p.items()}
    x = x0.to(dev)
    y = pkg.ssm_step(u.to(dev), d["A"], d["Bm"], d["C"], d["dt"], D.to(dev), x)
    torch.cuda.synchronize()
    ref, xr = _ref(u, p, D, x0.numpy().astype(np.complex128))
    err = rel_l2(to_np(y), ref)
    errx = rel_l2(x.cpu().numpy().astype(np.complex128), xr)
    say("  rel_l2=%.3e state=%.3e" % (err, errx))
    assert err <= TOL[io] and errx <= 1e-5


@pytest.mark.parametrize("io", ["f32", "f16", "bf16"])
def test_prefix_by_state_passing_then_decode(io):
    """Prompt through h3conv_state_pass (x_out), then token-by-token decode:
    together the full-length recurrence over prompt + generated tokens."""
    dev = device()
    B, H, S, T, N, K = 4, 6, 64, 512, 2048, 9
    say("prefix+decode io=%s B=%d H=%d S=%d prompt=%d (T=%d) decode=%d" % (io, B, H, S, N, T, K))
    g, p, D = _params(H, S, 77)
    u = wl.normal((B, H, N + K), g, dtype=DT[io])
    d = {k: v.to(dev) for k, v in p.items()}
    ud, Dd = u.to(dev), D.to(dev)
    y0, x = pkg.state_pass(ud[..., :N].contiguous(), d["A"], d["Bm"], d["C"], d["dt"], Dd, T, return_state=True)
    ys = [y0]
    for t in range(K):  # one token per call, as in generation
        ys.append(pkg.ssm_step(ud[..., N + t:N + t + 1].contiguous(), d["A"], d["Bm"], d["C"], d["dt"], Dd, x))
    torch.cuda.synchronize()
    got = np.concatenate([to_np(v) for v in ys], axis=-1)
    ref, xr = _ref(u, p, D, None)
    err, errx = rel_l2(got, ref), rel_l2(x.cpu().numpy().astype(np.complex128), xr)
    err_tail = rel_l2(got[..., N:], ref[..., N:])
    say("  rel_l2=%.3e generated-tokens=%.3e state=%.3e" % (err, err_tail, errx))
    assert err <= TOL[io] and err_tail <= TOL[io] and errx <= (1e-5 if io == "f32" else 1e-3)


def test_decode_generation_shape():
    """Generation at the pages' batch 64 (H3-125M width 768, 64 modes): a
    1024-token prompt by state passing, then 16 single-token steps; every
    row checked."""
    dev = device()
    B, H, S, T, N, K = 64, 768, 64, 1024, 1024, 16
    say("decode generation shape f16 B=%d H=%d S=%d prompt=%d decode=%d" % (B, H, S, N, K))
    g, p, D = _params(H, S, 1234)
    u = wl.normal((B, H, N + K), g, dtype=torch.float16)
    d = {k: v.to(dev) for k, v in p.items()}
    ud, Dd = u.to(dev), D.to(dev)
    _, x = pkg.state_pass(ud[..., :N].contiguous(), d["A"], d["Bm"], d["C"], d["dt"], Dd, T, return_state=True)
    ys = [pkg.ssm_step(ud[..., N + t:N + t + 1].contiguous(), d["A"], d["Bm"], d["C"], d["dt"], Dd, x)
          for t in range(K)]
    torch.cuda.synchronize()
    got = np.concatenate([to_np(v) for v in ys], axis=-1)
    ref, _ = _ref(u, p, D, None)
    ref = ref[..., N:]
    rows = row_rel_l2(got.reshape(B * H, K), ref.reshape(B * H, K))
    err = rel_l2(got, ref)
    say("  generated tokens rel_l2=%.3e max_row=%.3e" % (err, rows.max()))
    assert err <= TOL["f16"] and rows.max() <= TOL["f16"]
