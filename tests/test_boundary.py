"""Host-side checks of the C ABI (no GPU needed, no compute calls).

The library must load, export every entry point that include/h3conv.h
declares, and reject malformed arguments on the host before any HIP call.
Pointers handed to the rejecting calls are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import fft_long_convolution_flashconv_amd as pkg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3conv.h")

A16 = 0x10000       # fake, 16-byte aligned "device" addresses; never dereferenced
A16b = 0x20000
MIS = 0x10008       # misaligned


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(h3conv_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return pkg.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(pkg.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert pkg.load().h3conv_version() >= 100
    for s in range(6):
        assert pkg.status_string(s) and pkg.status_string(s) != "unknown status"
    assert pkg.status_string(99) == "unknown status"


def test_workspace_size(lib):
    assert pkg.workspace_size(pkg.OP_FFT_CONV, 8, 768, 1024) == 0
    # 16-bit H3 mix stages m and z channel-major as bf16: two [B, Dm, N] buffers
    assert pkg.workspace_size(pkg.OP_H3_MIX, 4, 2560, 2048) == 2 * 4 * 2560 * 2048 * 2
    n = pkg.workspace_size(pkg.OP_STATE_PASS, 2, 1024, 65536, 64, 8192)
    assert n > 0 and n % 256 == 0
    for bad in [(2, 4, 1000, 64, 8192), (2, 4, 8192, 65, 8192), (2, 4, 8192, 64, 100),
                (2, 4, 16384, 64, 16384), (2, 4, 8192, 64, 32)]:
        with pytest.raises(pkg.H3ConvError):
            pkg.workspace_size(pkg.OP_STATE_PASS, *bad)
    with pytest.raises(pkg.H3ConvError):
        pkg.workspace_size(7)


def _fc(lib, u=A16, f=A16b, D=0x30000, y=0x40000, B=2, H=3, N=64, io=1):
    return lib.h3conv_fft_conv(u, f, D, y, B, H, N, io, None)


def test_fft_conv_validation(lib):
    assert _fc(lib, B=-1) == pkg.ERR_INVALID_ARG
    assert _fc(lib, io=7) == pkg.ERR_INVALID_ARG
    assert _fc(lib, u=None) == pkg.ERR_INVALID_ARG
    assert _fc(lib, y=None) == pkg.ERR_INVALID_ARG
    assert _fc(lib, u=MIS) == pkg.ERR_INVALID_ARG
    assert _fc(lib, N=8193, io=0) == pkg.ERR_UNSUPPORTED      # fp32: 2N <= 16384
    assert _fc(lib, N=16385, io=1) == pkg.ERR_UNSUPPORTED     # 16-bit: 2N <= 32768
    # y overlapping u / f / D
    assert _fc(lib, y=A16 + 64) == pkg.ERR_INVALID_ARG
    assert _fc(lib, y=A16b) == pkg.ERR_INVALID_ARG
    # empty problems are no-ops even with NULL pointers
    assert _fc(lib, u=None, f=None, D=None, y=None, B=0) == pkg.OK
    assert _fc(lib, u=None, f=None, D=None, y=None, N=0) == pkg.OK


def test_ssm_filter_validation(lib):
    f = lib.h3conv_ssm_filter
    assert f(A16, A16b, 0x30000, 0x40000, 0x50000, 4, 0, 64, None) == pkg.ERR_INVALID_ARG
    assert f(A16, A16b, 0x30000, 0x40000, 0x50000, 4, 65, 64, None) == pkg.ERR_UNSUPPORTED
    assert f(None, A16b, 0x30000, 0x40000, 0x50000, 4, 8, 64, None) == pkg.ERR_INVALID_ARG
    assert f(A16, A16b, 0x30000, 0x40000, A16, 4, 8, 64, None) == pkg.ERR_INVALID_ARG  # f aliases A
    assert f(None, None, None, None, None, 0, 8, 64, None) == pkg.OK


def _sp(lib, u=0x100000, y=0x200000, x_in=None, x_out=None, ws=0x400000, ws_bytes=1 << 40,
        B=2, H=4, N=1024, S=8, T=256, io=1):
    return lib.h3conv_state_pass(u, 0x10000, 0x20000, 0x30000, 0x40000, 0x50000, x_in, x_out, y,
                                 B, H, N, S, T, io, ws, ws_bytes, None)


def test_state_pass_validation(lib):
    assert _sp(lib, N=1000) == pkg.ERR_UNSUPPORTED           # N % T != 0
    assert _sp(lib, T=96) == pkg.ERR_UNSUPPORTED             # T not a power of two
    assert _sp(lib, T=32) == pkg.ERR_UNSUPPORTED             # T below 64
    assert _sp(lib, T=16384, N=16384) == pkg.ERR_UNSUPPORTED  # chunk above the fused limit
    assert _sp(lib, S=65) == pkg.ERR_UNSUPPORTED
    assert _sp(lib, S=0) == pkg.ERR_INVALID_ARG
    assert _sp(lib, u=None) == pkg.ERR_INVALID_ARG
    assert _sp(lib, ws=None) == pkg.ERR_WORKSPACE
    assert _sp(lib, ws_bytes=16) == pkg.ERR_WORKSPACE
    assert _sp(lib, y=0x100000 + 128) == pkg.ERR_INVALID_ARG  # y overlaps u
    assert _sp(lib, x_out=0x200000) == pkg.ERR_INVALID_ARG    # x_out overlaps y
    assert _sp(lib, x_in=0x100008) == pkg.ERR_INVALID_ARG     # misaligned
    assert _sp(lib, B=0) == pkg.OK


def _hm(lib, out=0x900000, B=2, N=64, Dm=8, L=4, io=2, ws=0xa00000, nws=1 << 20):
    return lib.h3conv_h3_mix(0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000, out,
                             B, N, Dm, L, io, ws, nws, None)


def test_h3_mix_validation(lib):
    assert _hm(lib, L=0) == pkg.ERR_INVALID_ARG
    assert _hm(lib, L=5) == pkg.ERR_UNSUPPORTED
    assert _hm(lib, N=8193) == pkg.ERR_UNSUPPORTED
    assert _hm(lib, out=0x100000) == pkg.ERR_INVALID_ARG  # out aliases q
    assert _hm(lib, out=0x900008) == pkg.ERR_INVALID_ARG  # misaligned
    assert _hm(lib, ws=None) == pkg.ERR_WORKSPACE          # 16-bit path needs a workspace
    assert _hm(lib, nws=16) == pkg.ERR_WORKSPACE
    assert _hm(lib, ws=0x100000) == pkg.ERR_INVALID_ARG    # workspace overlaps q
    assert _hm(lib, B=0) == pkg.OK


def test_valid_call_without_device_reports_no_device(lib):
    """On a host with no HIP device a well-formed call returns NO_DEVICE, never crashes."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a HIP device is present; this host-only path is exercised on CPU machines")
    assert _fc(lib) == pkg.ERR_NO_DEVICE


def test_row_offset_limits_refused_before_any_hip_call(lib):
    """The 16-bit engine keeps row byte offsets of one launch within 32 bits:
    (2 SIG + 4) * 2 H N < 2^32 (SIG = 1 at N = 8192, so H <= 43690).  Larger
    H is refused on the host (UNSUPPORTED, not NO_DEVICE on a GPU-less host)."""
    assert _fc(lib, B=2, H=43691, N=8192, io=1) == pkg.ERR_UNSUPPORTED
    assert _fc(lib, B=2, H=43691, N=8192, io=2) == pkg.ERR_UNSUPPORTED
    # at N = 1024 (SIG = 4): 12 * 2 H * 1024 < 2^32  <=>  H <= 174762
    assert _fc(lib, B=2, H=174763, N=1024, io=1) == pkg.ERR_UNSUPPORTED
    # fp32 activations use 64-bit offsets
    r = _fc(lib, u=1 << 40, f=2 << 40, D=3 << 40, y=4 << 40, B=2, H=43691, N=8192, io=0)
    assert r in (pkg.ERR_NO_DEVICE, pkg.OK, pkg.ERR_HIP) and r != pkg.ERR_UNSUPPORTED
    # the H3 mix: B <= 65535 and the same row limit with H = Dm (16-bit)
    assert _hm(lib, B=65536, io=2) == pkg.ERR_UNSUPPORTED
    assert _hm(lib, N=8192, Dm=43691, io=1) == pkg.ERR_UNSUPPORTED


def test_state_pass_zero_length(lib):
    """N == 0: only x_out is written (a copy of x_in, or zeros); it is
    validated like any output."""
    assert _sp(lib, N=0) == pkg.OK                                     # no x_out: nothing to do
    assert _sp(lib, N=0, x_out=0x300008) == pkg.ERR_INVALID_ARG        # misaligned
    assert _sp(lib, N=0, x_in=0x300000, x_out=0x300000) == pkg.ERR_INVALID_ARG  # overlap
    import torch
    if torch.cuda.device_count() == 0:
        assert _sp(lib, N=0, x_out=0x300000) == pkg.ERR_NO_DEVICE


# ------------------------------------------------------------------ Python binding

def _cpu(*shape, dtype=None):
    import torch
    return torch.zeros(*shape, dtype=dtype or torch.float32)


def test_binding_checks_every_shape():
    """Every tensor's exact shape is checked before the C ABI is called (the
    library cannot see buffer sizes); CPU tensors of the right shapes are
    then refused for their device."""
    import torch
    h = torch.float16
    u = _cpu(2, 3, 64, dtype=h)
    with pytest.raises(ValueError, match="f must have shape"):
        pkg.fft_conv(u, _cpu(3, 63), _cpu(3))
    with pytest.raises(ValueError, match="D must have shape"):
        pkg.fft_conv(u, _cpu(3, 64), _cpu(4))
    with pytest.raises(ValueError, match="out must have shape"):
        pkg.fft_conv(u, _cpu(3, 64), _cpu(3), out=_cpu(2, 3, 32, dtype=h))
    with pytest.raises(ValueError, match="out must be"):
        pkg.fft_conv(u, _cpu(3, 64), _cpu(3), out=_cpu(2, 3, 64))
    with pytest.raises(ValueError, match="HIP device"):
        pkg.fft_conv(u, _cpu(3, 64), _cpu(3))
    A = _cpu(3, 8, 2)
    with pytest.raises(ValueError, match="Bm must have shape"):
        pkg.ssm_filter(A, _cpu(3, 7, 2), A.clone(), _cpu(3), 64)
    with pytest.raises(ValueError, match="dt must have shape"):
        pkg.ssm_filter(A, A.clone(), A.clone(), _cpu(4), 64)
    with pytest.raises(ValueError, match="out must have shape"):
        pkg.ssm_filter(A, A.clone(), A.clone(), _cpu(3), 64, out=_cpu(3, 65))
    with pytest.raises(ValueError, match="A must be"):
        pkg.state_pass(u, _cpu(4, 8, 2), A.clone(), A.clone(), _cpu(3), _cpu(3), 64)
    with pytest.raises(ValueError, match="C must have shape"):
        pkg.state_pass(u, A, A.clone(), _cpu(3, 8), _cpu(3), _cpu(3), 64)
    with pytest.raises(ValueError, match="x_in must have shape"):
        pkg.state_pass(u, A, A.clone(), A.clone(), _cpu(3), _cpu(3), 64, x_in=_cpu(2, 3, 7, 2))
    with pytest.raises(ValueError, match="D must have shape"):
        pkg.state_pass(u, A, A.clone(), A.clone(), _cpu(3), _cpu(2), 64)
    q = _cpu(2, 64, 5, dtype=h)
    with pytest.raises(ValueError, match="k must have shape"):
        pkg.h3_mix(q, _cpu(2, 64, 4, dtype=h), q.clone(), _cpu(5, 4), _cpu(5, 64), _cpu(5))
    with pytest.raises(ValueError, match="w must be"):
        pkg.h3_mix(q, q.clone(), q.clone(), _cpu(4, 4), _cpu(5, 64), _cpu(5))
    with pytest.raises(ValueError, match="f must have shape"):
        pkg.h3_mix(q, q.clone(), q.clone(), _cpu(5, 4), _cpu(5, 63), _cpu(5))
    with pytest.raises(ValueError, match="out must have shape"):
        pkg.h3_mix(q, q.clone(), q.clone(), _cpu(5, 4), _cpu(5, 64), _cpu(5), out=_cpu(2, 64, 6, dtype=h))
    with pytest.raises(ValueError, match="HIP device"):
        pkg.h3_mix(q, q.clone(), q.clone(), _cpu(5, 4), _cpu(5, 64), _cpu(5))


def test_ssm_step_validation(lib):
    f = lib.h3conv_ssm_step

    def call(u=0x100000, x=0x700000, y=0x800000, B=2, H=4, K=3, S=8, io=1):
        return f(u, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000, x, y, B, H, K, S, io, None)

    assert call(S=0) == pkg.ERR_INVALID_ARG
    assert call(S=65) == pkg.ERR_UNSUPPORTED
    assert call(K=-1) == pkg.ERR_INVALID_ARG
    assert call(u=None) == pkg.ERR_INVALID_ARG
    assert call(x=0x700008) == pkg.ERR_INVALID_ARG          # misaligned
    assert call(y=0x100000) == pkg.ERR_INVALID_ARG          # y aliases u
    assert call(x=0x200000) == pkg.ERR_INVALID_ARG          # x aliases A
    assert call(B=4, H=1 << 26) == pkg.ERR_UNSUPPORTED      # grid past 2^32 work-items
    assert call(B=(1 << 28) + 4, H=1) == pkg.ERR_UNSUPPORTED
    assert call(K=0, u=None, x=None, y=None) == pkg.OK      # empty: no-op


def test_fft_conv_bwd_validation(lib):
    f = lib.h3conv_fft_conv_bwd

    def call(u=0x100000, dy=0x200000, du=0x300000, df=0x400000, dD=0x500000, B=2, H=4, N=64, io=1):
        return f(u, 0x600000, 0x700000, dy, du, df, dD, B, H, N, io, None)

    assert call(io=9) == pkg.ERR_INVALID_ARG
    assert call(dy=None) == pkg.ERR_INVALID_ARG
    assert call(df=None) == pkg.ERR_INVALID_ARG
    assert call(du=0x300008) == pkg.ERR_INVALID_ARG        # misaligned
    assert call(du=0x200000) == pkg.ERR_INVALID_ARG        # du aliases dy
    assert call(dD=0x400000) == pkg.ERR_INVALID_ARG        # dD inside df
    assert call(N=8193) == pkg.ERR_UNSUPPORTED
    assert call(H=43691, N=8192, u=1 << 40, dy=2 << 40, du=3 << 40, df=4 << 40, dD=5 << 40) == pkg.ERR_UNSUPPORTED
    assert call(H=0) == pkg.OK


def test_h3_mix_mh_validation(lib):
    f = lib.h3conv_h3_mix_mh

    def call(out=0x900000, B=2, N=64, Dm=8, dh=2, L=4, io=2, ws=0xa00000, nws=1 << 20):
        return f(0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000, out, B, N, Dm, dh, L, io, ws, nws,
                 None)

    assert call(dh=0) == pkg.ERR_INVALID_ARG
    assert call(dh=3, Dm=9) == pkg.ERR_UNSUPPORTED      # not a power of two
    assert call(dh=64, Dm=64) == pkg.ERR_UNSUPPORTED    # above 32
    assert call(dh=4, Dm=6) == pkg.ERR_UNSUPPORTED      # does not divide Dm
    assert call(L=5) == pkg.ERR_UNSUPPORTED
    assert call(ws=None) == pkg.ERR_WORKSPACE
    assert call(nws=16) == pkg.ERR_WORKSPACE
    assert call(out=0x100000) == pkg.ERR_INVALID_ARG    # out aliases q
    assert call(B=0) == pkg.OK
    assert pkg.workspace_size(pkg.OP_H3_MIX_MH, 2, 8, 64, 2) == 2 * (2 * 64 * 8 * 2 * 2)


def test_noalloc_refuses_sizes_past_the_array(lib):
    """The entry point without a workspace refuses, before any HIP call,
    sizes whose workspace exceeds its static array, for every activation
    type (the pointers are fake and never touched)."""
    B, H, N, S, T = 2, 8192, 65536, 64, 8192
    # lower bounds of each type's workspace past the array: the 16-bit
    # projection tables alone (32 KiB per channel) and the fp32 chunk filter
    # alone (H * T * 4 bytes)
    assert H * 32768 > pkg.NOALLOC_WORKSPACE_BYTES
    assert H * T * 4 > pkg.NOALLOC_WORKSPACE_BYTES
    A = 1 << 36
    for io in (pkg.F16, pkg.BF16, pkg.F32):
        r = lib.h3conv_state_pass_noalloc(A, A + (1 << 30), A + (2 << 30), A + (3 << 30), A + (4 << 30),
                                          A + (5 << 30), None, None, A + (8 << 30), B, H, N, S, T, io, None)
        assert r == pkg.ERR_WORKSPACE
