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
    assert _fc(lib, N=8193) == pkg.ERR_UNSUPPORTED
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
