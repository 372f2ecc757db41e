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
  state_pass  chunked convolution with the diagonal-SSM state carried
              between chunks (exactly the full-length SSM; 16-bit activations
              pass the state every 64 samples, fp32 convolve chunks of T by FFT)
  h3_mix      out = q * (f * (shift(k) * v) + D * shift(k) * v)
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# H3CONV_LIB selects another build of the library (e.g. libh3conv_san.so,
# host code under AddressSanitizer, for host-only checks)
LIB_PATH = os.environ.get("H3CONV_LIB") or os.path.join(HERE, "libh3conv.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_NO_DEVICE, ERR_HIP, ERR_WORKSPACE = range(6)
F32, F16, BF16 = 0, 1, 2
OP_FFT_CONV, OP_STATE_PASS, OP_H3_MIX, OP_H3_MIX_MH = 0, 1, 2, 3
MAX_FUSED_N = 8192
MAX_FUSED_N_16BIT = 16384
MAX_STATE = 64

_IO = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
_lib = None

EXPORTS = ("h3conv_fft_conv", "h3conv_fft_conv_bidir", "h3conv_fft_conv_bwd", "h3conv_ssm_filter", "h3conv_state_pass", "h3conv_state_pass_noalloc",
           "h3conv_ssm_step", "h3conv_h3_mix", "h3conv_h3_mix_mh", "h3conv_workspace_size", "h3conv_status_string", "h3conv_version")
NOALLOC_WORKSPACE_BYTES = 128 * 1024 * 1024


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
    lib.h3conv_fft_conv_bidir.argtypes = [P, P, P, P, P, I64, I64, I64, I, P]
    lib.h3conv_fft_conv_bwd.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I, P]
    lib.h3conv_ssm_filter.argtypes = [P, P, P, P, P, I64, I64, I64, P]
    lib.h3conv_state_pass.argtypes = [P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I, P, SZ, P]
    lib.h3conv_state_pass_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I, P]
    lib.h3conv_ssm_step.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, I64, I, P]
    lib.h3conv_h3_mix.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, I, P, ctypes.c_size_t, P]
    lib.h3conv_h3_mix_mh.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I, P, SZ, P]
    lib.h3conv_workspace_size.argtypes = [I, I64, I64, I64, I64, I64]
    lib.h3conv_workspace_size.restype = SZ
    lib.h3conv_status_string.argtypes = [I]
    lib.h3conv_status_string.restype = ctypes.c_char_p
    lib.h3conv_version.restype = I
    for name in ("h3conv_fft_conv", "h3conv_fft_conv_bidir", "h3conv_fft_conv_bwd", "h3conv_ssm_filter", "h3conv_state_pass", "h3conv_state_pass_noalloc",
                 "h3conv_ssm_step", "h3conv_h3_mix", "h3conv_h3_mix_mh"):
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


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    """Type, dtype, exact shape and contiguity of one tensor argument (the
    device is checked for all arguments of a call together, by _same_device)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _same_device(**ts):
    """Every tensor on one HIP device, which is the current one (the library
    launches on the current device and its current stream)."""
    devs = {n: t.device for n, t in ts.items() if t is not None}
    for n, d in devs.items():
        if d.type != "cuda":
            raise ValueError("%s must be on a HIP device, got %s" % (n, d))
    if len(set(devs.values())) > 1:
        raise ValueError("all tensors must be on one device, got %s" % devs)
    d = next(iter(devs.values()))
    cur = torch.cuda.current_device()
    if d.index is not None and d.index != cur:
        raise ValueError("tensors are on %s but the current device is cuda:%d" % (d, cur))


def _cplx_param(t: torch.Tensor, name: str, shape=None) -> torch.Tensor:
    """Complex parameters are accepted as complex64 [...] or float32 [..., 2]."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.is_complex():
        if t.dtype != torch.complex64:
            raise ValueError("%s must be complex64 or float32 [..., 2], got %s" % (name, t.dtype))
        t = torch.view_as_real(t)
    _need(t, name, torch.float32, None if shape is None else tuple(shape) + (2,))
    if t.dim() < 1 or t.shape[-1] != 2:
        raise ValueError("%s must be complex or have a trailing dimension of 2" % name)
    return t


def _io(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _IO:
        raise ValueError("%s must be float32, float16 or bfloat16, got %s" % (name, t.dtype))
    return _IO[t.dtype]


def fft_conv(u: torch.Tensor, f: torch.Tensor, D: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """y[b,h,:] = causal (f[h] * u[b,h])[:N] + D[h] u[b,h]; u [B,H,N] f32/f16/bf16, f [H,N] f32, D [H] f32."""
    _need(u, "u")
    io = _io(u, "u")
    if u.dim() != 3:
        raise ValueError("u must be [B,H,N], got %s" % (tuple(u.shape),))
    B, H, N = u.shape
    _need(f, "f", torch.float32, (H, N)); _need(D, "D", torch.float32, (H,))
    if out is not None:
        _need(out, "out", u.dtype, (B, H, N))
    _same_device(u=u, f=f, D=D, out=out)
    y = torch.empty_like(u) if out is None else out
    _check(load().h3conv_fft_conv(_ptr(u), _ptr(f), _ptr(D), _ptr(y), B, H, N, io, _stream()),
           "h3conv_fft_conv")
    return y


def fft_conv_bidir(u: torch.Tensor, f: torch.Tensor, g: torch.Tensor, D: torch.Tensor,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """Bidirectional copies: y = causal (f * u) + anti-causal (g * u) + D u;
    u [B,H,N] f32/f16/bf16, f, g [H,N] f32, D [H] f32."""
    _need(u, "u")
    io = _io(u, "u")
    if u.dim() != 3:
        raise ValueError("u must be [B,H,N], got %s" % (tuple(u.shape),))
    B, H, N = u.shape
    _need(f, "f", torch.float32, (H, N)); _need(g, "g", torch.float32, (H, N)); _need(D, "D", torch.float32, (H,))
    if out is not None:
        _need(out, "out", u.dtype, (B, H, N))
    _same_device(u=u, f=f, g=g, D=D, out=out)
    y = torch.empty_like(u) if out is None else out
    _check(load().h3conv_fft_conv_bidir(_ptr(u), _ptr(f), _ptr(g), _ptr(D), _ptr(y), B, H, N, io, _stream()),
           "h3conv_fft_conv_bidir")
    return y


def fft_conv_bwd(u: torch.Tensor, f: torch.Tensor, D: torch.Tensor, dy: torch.Tensor, du=None, df=None, dD=None):
    """Gradients of y = fft_conv(u, f, D) for an upstream gradient dy.

    Returns (du [B,H,N] like u, df [H,N] f32, dD [H] f32); df and dD are
    summed over the batch."""
    _need(u, "u")
    io = _io(u, "u")
    if u.dim() != 3:
        raise ValueError("u must be [B,H,N], got %s" % (tuple(u.shape),))
    B, H, N = u.shape
    _need(f, "f", torch.float32, (H, N)); _need(D, "D", torch.float32, (H,))
    _need(dy, "dy", u.dtype, (B, H, N))
    if du is not None:
        _need(du, "du", u.dtype, (B, H, N))
    if df is not None:
        _need(df, "df", torch.float32, (H, N))
    if dD is not None:
        _need(dD, "dD", torch.float32, (H,))
    _same_device(u=u, f=f, D=D, dy=dy, du=du, df=df, dD=dD)
    du = torch.empty_like(u) if du is None else du
    df = torch.empty(H, N, device=u.device, dtype=torch.float32) if df is None else df
    dD = torch.empty(H, device=u.device, dtype=torch.float32) if dD is None else dD
    _check(load().h3conv_fft_conv_bwd(_ptr(u), _ptr(f), _ptr(D), _ptr(dy), _ptr(du), _ptr(df), _ptr(dD),
                                       B, H, N, io, _stream()),
           "h3conv_fft_conv_bwd")
    return du, df, dD


def ssm_filter(A: torch.Tensor, Bm: torch.Tensor, C: torch.Tensor, dt: torch.Tensor, N: int,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """f[h,k] = 2 Re(sum_j C exp(dt A k) dt B), k < N; A, Bm, C [H,S] complex, dt [H] f32."""
    A = _cplx_param(A, "A")
    if A.dim() != 3:
        raise ValueError("A must be [H,S] complex")
    H, S = A.shape[0], A.shape[1]
    Bm = _cplx_param(Bm, "Bm", (H, S)); C = _cplx_param(C, "C", (H, S))
    _need(dt, "dt", torch.float32, (H,))
    if out is not None:
        _need(out, "out", torch.float32, (H, int(N)))
    _same_device(A=A, Bm=Bm, C=C, dt=dt, out=out)
    f = torch.empty(H, int(N), device=A.device, dtype=torch.float32) if out is None else out
    _check(load().h3conv_ssm_filter(_ptr(A), _ptr(Bm), _ptr(C), _ptr(dt), _ptr(f), H, S, int(N), _stream()),
           "h3conv_ssm_filter")
    return f


def _sp_args(u, A, Bm, C, dt, D, x_in, out, workspace):
    _need(u, "u")
    io = _io(u, "u")
    if u.dim() != 3:
        raise ValueError("u must be [B,H,N], got %s" % (tuple(u.shape),))
    B, H, N = u.shape
    A = _cplx_param(A, "A")
    if A.dim() != 3 or A.shape[0] != H:
        raise ValueError("A must be [H,S] complex with H = %d, got %s" % (H, tuple(A.shape)))
    S = A.shape[1]
    Bm = _cplx_param(Bm, "Bm", (H, S)); C = _cplx_param(C, "C", (H, S))
    _need(dt, "dt", torch.float32, (H,)); _need(D, "D", torch.float32, (H,))
    if x_in is not None:
        x_in = _cplx_param(x_in, "x_in", (B, H, S))
    if out is not None:
        _need(out, "out", u.dtype, (B, H, N))
    if workspace is not None:
        _need(workspace, "workspace")
    _same_device(u=u, A=A, Bm=Bm, C=C, dt=dt, D=D, x_in=x_in, out=out, workspace=workspace)
    return io, B, H, N, S, A, Bm, C, x_in


def state_pass(u, A, Bm, C, dt, D, T: int, x_in=None, return_state: bool = False,
               out=None, workspace=None):
    """Full-length diagonal SSM over u [B,H,N] by chunks of T (state carried between chunks).

    Returns y, or (y, x_out) with x_out [B,H,S] complex64 if ``return_state``.
    """
    io, B, H, N, S, A, Bm, C, x_in = _sp_args(u, A, Bm, C, dt, D, x_in, out, workspace)
    y = torch.empty_like(u) if out is None else out
    x_out = torch.empty(B, H, S, 2, device=u.device, dtype=torch.float32) if return_state else None
    need = workspace_size(OP_STATE_PASS, B, H, N, S, T) if N > 0 else 0
    ws = workspace
    if ws is None or ws.numel() * ws.element_size() < need:
        ws = torch.empty(max(need, 1), device=u.device, dtype=torch.uint8)
    _check(load().h3conv_state_pass(_ptr(u), _ptr(A), _ptr(Bm), _ptr(C), _ptr(dt), _ptr(D), _ptr(x_in),
                                     _ptr(x_out), _ptr(y), B, H, N, S, int(T), io, _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream()),
           "h3conv_state_pass")
    if return_state:
        return y, torch.view_as_complex(x_out)
    return y


def state_pass_noalloc(u, A, Bm, C, dt, D, T: int, out, x_in=None, x_out=None):
    """state_pass through h3conv_state_pass_noalloc: no workspace, no device
    allocation in the library or here (``out``, and ``x_out`` [B,H,S,2]
    float32 if the final state is wanted, are the caller's).  The library's
    static scratch array of NOALLOC_WORKSPACE_BYTES per device is shared by
    all such calls on a device: calls that overlap in time race."""
    io, B, H, N, S, A, Bm, C, x_in = _sp_args(u, A, Bm, C, dt, D, x_in, out, None)
    if out is None:
        raise ValueError("out is required (this entry point allocates nothing)")
    if x_out is not None:
        x_out = _cplx_param(x_out, "x_out", (B, H, S))
        _same_device(u=u, x_out=x_out)
    _check(load().h3conv_state_pass_noalloc(_ptr(u), _ptr(A), _ptr(Bm), _ptr(C), _ptr(dt), _ptr(D),
                                             _ptr(x_in), _ptr(x_out), _ptr(out), B, H, N, S, int(T), io,
                                             _stream()),
           "h3conv_state_pass_noalloc")
    return out


def ssm_step(u, A, Bm, C, dt, D, x, out=None):
    """K recurrent steps per row: x <- exp(dt A) x + dt B u_t, y_t = 2 Re(C.x) + D u_t.

    u [B,H,K] f32/f16/bf16; A, Bm, C [H,S] complex; dt, D [H]; x [B,H,S]
    complex64 (or float32 [B,H,S,2]), updated in place.  Returns y [B,H,K]."""
    _need(u, "u")
    io = _io(u, "u")
    if u.dim() != 3:
        raise ValueError("u must be [B,H,K], got %s" % (tuple(u.shape),))
    B, H, K = u.shape
    A = _cplx_param(A, "A")
    if A.dim() != 3 or A.shape[0] != H:
        raise ValueError("A must be [H,S] complex with H = %d, got %s" % (H, tuple(A.shape)))
    S = A.shape[1]
    Bm = _cplx_param(Bm, "Bm", (H, S)); C = _cplx_param(C, "C", (H, S))
    _need(dt, "dt", torch.float32, (H,)); _need(D, "D", torch.float32, (H,))
    xv = _cplx_param(x, "x", (B, H, S))
    if out is not None:
        _need(out, "out", u.dtype, (B, H, K))
    _same_device(u=u, A=A, Bm=Bm, C=C, dt=dt, D=D, x=xv, out=out)
    y = torch.empty_like(u) if out is None else out
    _check(load().h3conv_ssm_step(_ptr(u), _ptr(A), _ptr(Bm), _ptr(C), _ptr(dt), _ptr(D), _ptr(xv), _ptr(y),
                                   B, H, K, S, io, _stream()),
           "h3conv_ssm_step")
    return y


def h3_mix(q, k, v, w, f, D, out=None, workspace=None):
    """out = q * ((f * m)[:N] + D m), m = shift(k) * v; q,k,v [B,N,Dm], w [Dm,L], f [Dm,N], D [Dm].

    16-bit activations stage m and z channel-major in a workspace
    (allocated here when not given)."""
    _need(q, "q")
    io = _io(q, "q")
    if q.dim() != 3:
        raise ValueError("q must be [B,N,Dm], got %s" % (tuple(q.shape),))
    B, N, Dm = q.shape
    _need(k, "k", q.dtype, (B, N, Dm)); _need(v, "v", q.dtype, (B, N, Dm))
    _need(w, "w", torch.float32)
    if w.dim() != 2 or w.shape[0] != Dm:
        raise ValueError("w must be [Dm,L] with Dm = %d, got %s" % (Dm, tuple(w.shape)))
    L = w.shape[1]
    _need(f, "f", torch.float32, (Dm, N)); _need(D, "D", torch.float32, (Dm,))
    if out is not None:
        _need(out, "out", q.dtype, (B, N, Dm))
    if workspace is not None:
        _need(workspace, "workspace")
    _same_device(q=q, k=k, v=v, w=w, f=f, D=D, out=out, workspace=workspace)
    o = torch.empty_like(q) if out is None else out
    ws, nws = None, 0
    if q.dtype != torch.float32:
        ws = workspace if workspace is not None else torch.empty(
            max(workspace_size(OP_H3_MIX, B, Dm, N), 1), dtype=torch.uint8, device=q.device)
        nws = ws.numel() * ws.element_size()
    _check(load().h3conv_h3_mix(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(f), _ptr(D), _ptr(o), B, N, Dm, L,
                                io, _ptr(ws) if ws is not None else None, nws, _stream()),
           "h3conv_h3_mix")
    return o


def h3_mix_mh(q, k, v, w, f, D, dh: int, out=None, workspace=None):
    """Multi-head H3 mixing, head dimension dh: per head, m = shift(k)^T v
    (outer product), z = (f * m)[:N] + D m per state entry, out_j = sum_i q_i z_ij.
    q, k, v [B,N,Dm]; w [Dm,L]; f [Dm*dh, N]; D [Dm*dh].  The workspace (two
    channel-major stagings of the B x Dm*dh state rows) is allocated here
    when not given."""
    _need(q, "q")
    io = _io(q, "q")
    if q.dim() != 3:
        raise ValueError("q must be [B,N,Dm], got %s" % (tuple(q.shape),))
    B, N, Dm = q.shape
    dh = int(dh)
    if dh < 1 or Dm % dh != 0:
        raise ValueError("dh must divide Dm = %d" % Dm)
    _need(k, "k", q.dtype, (B, N, Dm)); _need(v, "v", q.dtype, (B, N, Dm))
    _need(w, "w", torch.float32)
    if w.dim() != 2 or w.shape[0] != Dm:
        raise ValueError("w must be [Dm,L] with Dm = %d, got %s" % (Dm, tuple(w.shape)))
    L = w.shape[1]
    _need(f, "f", torch.float32, (Dm * dh, N)); _need(D, "D", torch.float32, (Dm * dh,))
    if out is not None:
        _need(out, "out", q.dtype, (B, N, Dm))
    if workspace is not None:
        _need(workspace, "workspace")
    _same_device(q=q, k=k, v=v, w=w, f=f, D=D, out=out, workspace=workspace)
    o = torch.empty_like(q) if out is None else out
    need = workspace_size(OP_H3_MIX_MH, B, Dm, N, dh) * (2 if io == F32 else 1)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(load().h3conv_h3_mix_mh(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(f), _ptr(D), _ptr(o), B, N, Dm, dh, L,
                                   io, _ptr(ws), ws.numel() * ws.element_size(), _stream()),
           "h3conv_h3_mix_mh")
    return o
