"""Python binding of the gfx950 causal SSM long-convolution library (libh3conv.so).

Thin ctypes marshalling over the C ABI declared in ``include/h3conv.h``: the
functions here check dtype, device and contiguity of torch tensors, pass raw
device pointers and the current HIP stream, and turn status codes into
exceptions.  Every step of the computation runs in the HIP kernels; there is no
host or PyTorch fallback, and importing the binding fails loudly if the
library has not been built.

Operations (after "Hungry Hungry Hippos: Towards Language Modeling with State
Space Models"):
  fft_conv    y = (f * u)[:N] + D u, fused FFT convolution per channel
  ssm_filter  f_k = 2 Re(sum_j C_j exp(dt A_j k) dt B_j)
  state_pass  chunked FFT convolution with the diagonal-SSM state carried
              between chunks (exactly the full-length SSM)
  h3_mix      out = q * (f * (shift(k) * v) + D * shift(k) * v)
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libh3conv.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_NO_DEVICE, ERR_HIP, ERR_WORKSPACE = range(6)
F32, F16, BF16 = 0, 1, 2
OP_FFT_CONV, OP_STATE_PASS, OP_H3_MIX = 0, 1, 2
MAX_FUSED_N = 8192
MAX_STATE = 64

_IO = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
_lib = None

EXPORTS = ("h3conv_fft_conv", "h3conv_ssm_filter", "h3conv_state_pass", "h3conv_h3_mix",
           "h3conv_workspace_size", "h3conv_status_string", "h3conv_version")


class H3ConvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libh3conv.so (built by ``build.py``); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libh3conv.so not built: run `python fft_long_convolution_flashconv_amd/build.py` "
                           "(looked for %s)" % path)
    lib = ctypes.CDLL(path)
    P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.h3conv_fft_conv.argtypes = [P, P, P, P, I64, I64, I64, I, P]
    lib.h3conv_ssm_filter.argtypes = [P, P, P, P, P, I64, I64, I64, P]
    lib.h3conv_state_pass.argtypes = [P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I, P, SZ, P]
    lib.h3conv_h3_mix.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, I, P, ctypes.c_size_t, P]
    lib.h3conv_workspace_size.argtypes = [I, I64, I64, I64, I64, I64]
    lib.h3conv_workspace_size.restype = SZ
    lib.h3conv_status_string.argtypes = [I]
    lib.h3conv_status_string.restype = ctypes.c_char_p
    lib.h3conv_version.restype = I
    for name in ("h3conv_fft_conv", "h3conv_ssm_filter", "h3conv_state_pass", "h3conv_h3_mix"):
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().h3conv_status_string(int(status)).decode()


def workspace_size(op: int, B: int = 0, H: int = 0, N: int = 0, S: int = 0, T: int = 0) -> int:
    n = load().h3conv_workspace_size(int(op), int(B), int(H), int(N), int(S), int(T))
    if n == ctypes.c_size_t(-1).value:
        raise H3ConvError(ERR_UNSUPPORTED, "workspace_size")
    return int(n)


def _check(status: int, where: str) -> None:
    if status != OK:
        raise H3ConvError(status, where)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a HIP device" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))


def _cplx_param(t: torch.Tensor, name: str) -> torch.Tensor:
    """Complex parameters are accepted as complex64 [...] or float32 [..., 2]."""
    if t.is_complex():
        t = torch.view_as_real(t)
    _need(t, name, torch.float32)
    if t.shape[-1] != 2:
        raise ValueError("%s must be complex or have a trailing dimension of 2" % name)
    return t


def fft_conv(u: torch.Tensor, f: torch.Tensor, D: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """y[b,h,:] = causal (f[h] * u[b,h])[:N] + D[h] u[b,h]; u [B,H,N] f32/f16/bf16, f [H,N] f32, D [H] f32."""
    _need(u, "u")
    if u.dtype not in _IO:
        raise ValueError("u must be float32, float16 or bfloat16")
    B, H, N = u.shape
    _need(f, "f", torch.float32); _need(D, "D", torch.float32)
    if tuple(f.shape) != (H, N) or tuple(D.shape) != (H,):
        raise ValueError("f must be [H,N] and D [H]")
    y = torch.empty_like(u) if out is None else out
    _need(y, "out", u.dtype)
    _check(load().h3conv_fft_conv(_ptr(u), _ptr(f), _ptr(D), _ptr(y), B, H, N, _IO[u.dtype], _stream()),
           "h3conv_fft_conv")
    return y


def ssm_filter(A: torch.Tensor, Bm: torch.Tensor, C: torch.Tensor, dt: torch.Tensor, N: int,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """f[h,k] = 2 Re(sum_j C exp(dt A k) dt B), k < N; A, Bm, C [H,S] complex, dt [H] f32."""
    A = _cplx_param(A, "A"); Bm = _cplx_param(Bm, "Bm"); C = _cplx_param(C, "C")
    _need(dt, "dt", torch.float32)
    H, S = A.shape[0], A.shape[1]
    f = torch.empty(H, N, device=A.device, dtype=torch.float32) if out is None else out
    _need(f, "out", torch.float32)
    _check(load().h3conv_ssm_filter(_ptr(A), _ptr(Bm), _ptr(C), _ptr(dt), _ptr(f), H, S, int(N), _stream()),
           "h3conv_ssm_filter")
    return f


def state_pass(u, A, Bm, C, dt, D, T: int, x_in=None, return_state: bool = False,
               out=None, workspace=None):
    """Full-length diagonal SSM over u [B,H,N] by chunks of T (state carried between chunks).

    Returns y, or (y, x_out) with x_out [B,H,S] complex64 if ``return_state``.
    """
    _need(u, "u")
    if u.dtype not in _IO:
        raise ValueError("u must be float32, float16 or bfloat16")
    A = _cplx_param(A, "A"); Bm = _cplx_param(Bm, "Bm"); C = _cplx_param(C, "C")
    _need(dt, "dt", torch.float32); _need(D, "D", torch.float32)
    B, H, N = u.shape
    S = A.shape[1]
    if x_in is not None:
        x_in = _cplx_param(x_in, "x_in")
    y = torch.empty_like(u) if out is None else out
    _need(y, "out", u.dtype)
    x_out = torch.empty(B, H, S, 2, device=u.device, dtype=torch.float32) if return_state else None
    need = workspace_size(OP_STATE_PASS, B, H, N, S, T)
    ws = workspace
    if ws is None or ws.numel() * ws.element_size() < need:
        ws = torch.empty(max(need, 1), device=u.device, dtype=torch.uint8)
    _check(load().h3conv_state_pass(_ptr(u), _ptr(A), _ptr(Bm), _ptr(C), _ptr(dt), _ptr(D), _ptr(x_in),
                                     _ptr(x_out), _ptr(y), B, H, N, S, int(T), _IO[u.dtype], _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream()),
           "h3conv_state_pass")
    if return_state:
        return y, torch.view_as_complex(x_out)
    return y


def h3_mix(q, k, v, w, f, D, out=None, workspace=None):
    """out = q * ((f * m)[:N] + D m), m = shift(k) * v; q,k,v [B,N,Dm], w [Dm,L], f [Dm,N], D [Dm].

    16-bit activations stage m and z channel-major in a workspace
    (allocated here when not given)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    if q.dtype not in _IO:
        raise ValueError("q, k, v must be float32, float16 or bfloat16")
    B, N, Dm = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    _need(w, "w", torch.float32); _need(f, "f", torch.float32); _need(D, "D", torch.float32)
    L = w.shape[1]
    o = torch.empty_like(q) if out is None else out
    _need(o, "out", q.dtype)
    ws, nws = None, 0
    if q.dtype != torch.float32:
        ws = workspace if workspace is not None else torch.empty(
            workspace_size(OP_H3_MIX, B, Dm, N), dtype=torch.uint8, device=q.device)
        nws = ws.numel() * ws.element_size()
    _check(load().h3conv_h3_mix(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(f), _ptr(D), _ptr(o), B, N, Dm, L,
                                _IO[q.dtype], _ptr(ws) if ws is not None else None, nws, _stream()),
           "h3conv_h3_mix")
    return o
