"""fp64 CPU oracle for the causal SSM long convolution (H3 / FlashConv).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this module; the GPU library and
its Python binding never do, and this module imports nothing from them.

The arithmetic lives in ``h3conv_oracle.c`` (plain C, fp64, OpenMP over
independent rows).  This wrapper only converts arrays to contiguous float64
and calls it.  Each function states the definition it computes and the
passage of the pages it follows; see the C file for the full list of readings.

Parity pins (tests/test_oracle.py) tie every function here to something other
than itself: exact integer brute force, a library convolution, closed forms,
identity/delta/impulse cases, linearity, and the filter-vs-recurrence
equality the pages state.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "h3conv_oracle.c")
# H3CONV_ORACLE_SANITIZE=1 builds and loads a copy instrumented with
# AddressSanitizer and UndefinedBehaviorSanitizer (the process must preload
# gcc's libasan, e.g. LD_PRELOAD=$(gcc -print-file-name=libasan.so)).
_SANITIZE = os.environ.get("H3CONV_ORACLE_SANITIZE") == "1"
_LIB = os.path.join(_HERE, "liboracle_san.so" if _SANITIZE else "liboracle.so")
_lib = None

MAX_STATE = 256  # per-row state buffer size of oracle_ssm_recurrence


def build(force: bool = False) -> str:
    """Compile the oracle shared library with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        if _SANITIZE:
            cmd[1:1] = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.oracle_causal_conv.argtypes = [P, P, P, P, I, I, I]
        lib.oracle_causal_conv_bwd.argtypes = [P, P, P, P, P, P, P, I, I, I]
        lib.oracle_bidir_conv.argtypes = [P, P, P, P, P, I, I, I]
        lib.oracle_h3_mix_mh.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P]
        lib.oracle_ssm_filter.argtypes = [P, P, P, P, P, I, I, I]
        lib.oracle_ssm_recurrence.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I]
        lib.oracle_h3_mix.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P]
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        for fn in (lib.oracle_causal_conv, lib.oracle_causal_conv_bwd, lib.oracle_bidir_conv, lib.oracle_h3_mix_mh,
                   lib.oracle_ssm_filter,
                   lib.oracle_ssm_recurrence, lib.oracle_h3_mix):
            fn.restype = None
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # a torch tensor
        a = a.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _cplx(a) -> np.ndarray:
    """Complex array -> interleaved (re, im) float64, trailing dim 2."""
    if hasattr(a, "detach"):
        a = a.detach().cpu()
        if a.is_complex():
            a = a.to(dtype=__import__("torch").complex128).numpy()
        else:
            a = a.double().numpy()
    a = np.asarray(a)
    if np.iscomplexobj(a):
        a = np.stack([a.real, a.imag], axis=-1)
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def causal_conv(u, f, D) -> np.ndarray:
    """y[b,h,t] = sum_{k<=t} f[h,t-k] u[b,h,k] + D[h] u[b,h,t] (fp64).

    u: [B,H,N]; f: [H,N]; D: [H].  The causal linear convolution with residual
    of the summary page, section 2 "Convolutional view", truncated to the
    first N outputs as in Appendix C.1.
    """
    u = _f64(u); f = _f64(f); D = _f64(D)
    B, H, N = u.shape
    assert f.shape == (H, N) and D.shape == (H,)
    y = np.empty_like(u)
    _load().oracle_causal_conv(_ptr(u), _ptr(f), _ptr(D), _ptr(y), B, H, N)
    return y


def bidir_conv(u, f, g, D) -> np.ndarray:
    """y[b,h,t] = sum_{k<=t} f[h,t-k] u[b,h,k] + sum_{k>=t} g[h,k-t] u[b,h,k] + D[h] u[b,h,t] (fp64).

    u: [B,H,N]; f, g: [H,N]; D: [H].  The layer as bidirectional copies (the
    summary page, E.4): a causal and an anti-causal convolution, summed, with
    one residual.
    """
    u = _f64(u); f = _f64(f); g = _f64(g); D = _f64(D)
    B, H, N = u.shape
    assert f.shape == (H, N) and g.shape == (H, N) and D.shape == (H,)
    y = np.empty_like(u)
    _load().oracle_bidir_conv(_ptr(u), _ptr(f), _ptr(g), _ptr(D), _ptr(y), B, H, N)
    return y


def causal_conv_bwd(u, f, D, dy):
    """Gradients (du, df, dD) of y = causal_conv(u, f, D) for upstream dy (fp64):

      du[b,h,k] = sum_{t>=k} f[h,t-k] dy[b,h,t] + D[h] dy[b,h,k]
      df[h,s]   = sum_b sum_{t>=s} dy[b,h,t] u[b,h,t-s]
      dD[h]     = sum_b sum_t dy[b,h,t] u[b,h,t]

    u, dy: [B,H,N]; f: [H,N]; D: [H].  The backward pass of the summary
    page's Appendix C.1: correlations with the filter and with the input,
    D*dy entering du.
    """
    u = _f64(u); f = _f64(f); D = _f64(D); dy = _f64(dy)
    B, H, N = u.shape
    assert dy.shape == u.shape and f.shape == (H, N) and D.shape == (H,)
    du = np.empty_like(u)
    df = np.empty((H, N), dtype=np.float64)
    dD = np.empty(H, dtype=np.float64)
    _load().oracle_causal_conv_bwd(_ptr(u), _ptr(f), _ptr(D), _ptr(dy), _ptr(du), _ptr(df), _ptr(dD), B, H, N)
    return du, df, dD


def ssm_filter(A, Bm, C, dt, N: int) -> np.ndarray:
    """f[h,k] = 2 Re(sum_j C_j exp(dt A_j k) dt B_j), k < N (fp64).

    A, Bm, C: [H,S] complex (or [H,S,2] interleaved); dt: [H].  The filter
    f = [CB, CAB, CA^2B, ...] of the blog's section "The Convolution
    Connection" with Abar = exp(dt A), Bbar = dt B.
    """
    A = _cplx(A); Bm = _cplx(Bm); C = _cplx(C); dt = _f64(dt)
    H, S = A.shape[:2]
    f = np.empty((H, N), dtype=np.float64)
    _load().oracle_ssm_filter(_ptr(A), _ptr(Bm), _ptr(C), _ptr(dt), _ptr(f), H, S, int(N))
    return f


def ssm_recurrence(u, A, Bm, C, dt, D, x_in=None, return_state: bool = False):
    """Step-by-step diagonal SSM: x <- exp(dt A) x + dt B u_t,
    y_t = 2 Re(C.x) + D u_t (fp64).

    u: [B,H,N]; A, Bm, C: [H,S] complex; dt, D: [H]; x_in: [B,H,S] complex or
    None (zero state).  Returns y, or (y, x_out) with x_out [B,H,S] complex128.
    """
    u = _f64(u); A = _cplx(A); Bm = _cplx(Bm); C = _cplx(C)
    dt = _f64(dt); D = _f64(D)
    B, H, N = u.shape
    S = A.shape[1]
    if S > MAX_STATE:
        raise ValueError("oracle recurrence supports at most %d modes" % MAX_STATE)
    xin = None if x_in is None else _cplx(x_in)
    y = np.empty_like(u)
    xo = np.empty((B, H, S, 2), dtype=np.float64) if return_state else None
    _load().oracle_ssm_recurrence(
        _ptr(u), _ptr(A), _ptr(Bm), _ptr(C), _ptr(dt), _ptr(D),
        None if xin is None else _ptr(xin), _ptr(y),
        None if xo is None else _ptr(xo), B, H, N, S)
    if return_state:
        return y, xo[..., 0] + 1j * xo[..., 1]
    return y


def h3_mix(q, k, v, w, f, D) -> np.ndarray:
    """out = q (.) ( causal_conv(shift(k) (.) v, f) + D (.) (shift(k) (.) v) ).

    q, k, v: [B,N,Dm] (channel last); w: [Dm,L] shift taps (w[:,0] on k_t);
    f: [Dm,N]; D: [Dm].  The H3 composition of the blog's section "The
    Solution, Part 1" with head dimension 1.
    """
    q = _f64(q); k = _f64(k); v = _f64(v); w = _f64(w); f = _f64(f); D = _f64(D)
    B, N, Dm = q.shape
    L = w.shape[1]
    out = np.empty_like(q)
    scratch = np.empty(2 * N * max(1, max_threads()), dtype=np.float64)
    _load().oracle_h3_mix(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(f), _ptr(D),
                          _ptr(out), B, N, Dm, L, _ptr(scratch))
    return out


def h3_mix_mh(q, k, v, w, f, D, dh: int) -> np.ndarray:
    """Multi-head H3 mixing with head dimension dh (fp64): per head, the
    outer product of shift(k) and v, a long convolution of every entry
    (i, j) with its own filter f[(h*dh+i)*dh+j] and D, then out_j = sum_i
    q_i z_ij.  q, k, v: [B,N,Dm]; w: [Dm,L]; f: [Dm*dh,N]; D: [Dm*dh].  The
    summary page's section 3 and Appendix C (keys in separate heads); dh = 1
    is h3_mix.
    """
    q = _f64(q); k = _f64(k); v = _f64(v); w = _f64(w); f = _f64(f); D = _f64(D)
    B, N, Dm = q.shape
    L = w.shape[1]
    assert Dm % dh == 0 and f.shape == (Dm * dh, N) and D.shape == (Dm * dh,) and w.shape[0] == Dm
    out = np.empty_like(q)
    scratch = np.empty((2 * dh * dh + dh) * N * max(1, max_threads()), dtype=np.float64)
    _load().oracle_h3_mix_mh(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(f), _ptr(D), _ptr(out),
                             B, N, Dm, int(dh), L, _ptr(scratch))
    return out
