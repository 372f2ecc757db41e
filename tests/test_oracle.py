"""Pins of the fp64 CPU oracle against facts fixed outside the oracle itself.

Each test ties one oracle function to something it cannot share a mistake
with: hand-worked golden values, exact integer brute force, a library
convolution or IIR filter, closed forms, delta/impulse identities, linearity,
and the equality of the convolutional and recurrent views of an SSM that the
pages state.  No GPU is used.
"""
import math
import os

import numpy as np
import pytest
import scipy.signal

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = np.array([float(x) for x in v.split()], dtype=np.float64)
    return out


def _rel(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


def _rand_ssm(rng, H, S, dt_lo=1e-3, dt_hi=1e-1):
    A = -rng.uniform(0.05, 1.0, size=(H, S)) + 1j * math.pi * rng.integers(0, 64, size=(H, S))
    Bm = rng.standard_normal((H, S)) + 1j * rng.standard_normal((H, S))
    C = rng.standard_normal((H, S)) + 1j * rng.standard_normal((H, S))
    dt = np.exp(rng.uniform(math.log(dt_lo), math.log(dt_hi), size=H))
    return A, Bm, C, dt


# ---------------------------------------------------------------- golden

def test_golden_causal_conv():
    g = _read_golden("causal_conv_hand.txt")
    for case in ("case1", "case2"):
        u = g[case + "_u"][None, None, :]
        f = g[case + "_f"][None, :]
        D = g[case + "_D"]
        y = oracle.causal_conv(u, f, D)
        assert np.array_equal(y[0, 0], g[case + "_y"]), case


def test_golden_ssm():
    g = _read_golden("ssm_hand.txt")
    cases = {"sum": (0.0 + 0.0j), "alt": (0.0 + 1j * math.pi)}
    for case, a in cases.items():
        A = np.array([[a]]); Bm = np.array([[1.0 + 0j]]); C = np.array([[0.5 + 0j]])
        dt = np.array([1.0]); D = g[case + "_D"]
        u = g[case + "_u"][None, None, :]
        y = oracle.ssm_recurrence(u, A, Bm, C, dt, D)
        np.testing.assert_allclose(y[0, 0], g[case + "_y"], rtol=0, atol=1e-14)
        f = oracle.ssm_filter(A, Bm, C, dt, u.shape[-1])
        np.testing.assert_allclose(f[0], g[case + "_f"], rtol=0, atol=1e-14)


def test_golden_h3_mix():
    g = _read_golden("h3_mix_hand.txt")
    q, k, v = (g[x][None, :, None] for x in ("q", "k", "v"))
    w = g["w"][None, :]
    for case in ("case1", "case2"):
        out = oracle.h3_mix(q, k, v, w, g[case + "_f"][None, :], g[case + "_D"])
        assert np.array_equal(out[0, :, 0], g[case + "_out"]), case


# ---------------------------------------------------------------- causal_conv

@pytest.mark.parametrize("N", [1, 2, 5, 17, 64])
def test_causal_conv_bruteforce_exact(N):
    """Small integers make fp64 exact: compare bitwise with an integer Toeplitz product."""
    rng = np.random.default_rng(N)
    B, H = 2, 3
    u = rng.integers(-8, 9, size=(B, H, N))
    f = rng.integers(-8, 9, size=(H, N))
    D = rng.integers(-4, 5, size=H)
    y = oracle.causal_conv(u.astype(float), f.astype(float), D.astype(float))
    for b in range(B):
        for h in range(H):
            T = [[int(f[h, t - k]) if k <= t else 0 for k in range(N)] for t in range(N)]
            ref = [sum(T[t][k] * int(u[b, h, k]) for k in range(N)) + int(D[h]) * int(u[b, h, t])
                   for t in range(N)]
            assert y[b, h].tolist() == [float(x) for x in ref]


def test_causal_conv_vs_numpy_convolve():
    rng = np.random.default_rng(1)
    B, H, N = 2, 3, 300
    u = rng.standard_normal((B, H, N)); f = rng.standard_normal((H, N)); D = rng.standard_normal(H)
    y = oracle.causal_conv(u, f, D)
    for b in range(B):
        for h in range(H):
            ref = np.convolve(u[b, h], f[h])[:N] + D[h] * u[b, h]
            assert _rel(y[b, h], ref) < 1e-13


def test_causal_conv_linearity():
    rng = np.random.default_rng(2)
    B, H, N = 2, 2, 200
    u1, u2 = rng.standard_normal((2, B, H, N)); f1, f2 = rng.standard_normal((2, H, N))
    D = rng.standard_normal(H); a, b = 0.75, -1.5
    y = oracle.causal_conv(a * u1 + b * u2, f1, D)
    ref = a * oracle.causal_conv(u1, f1, D) + b * oracle.causal_conv(u2, f1, D)
    assert _rel(y, ref) < 1e-13
    z0 = np.zeros(H)
    y = oracle.causal_conv(u1, a * f1 + b * f2, z0)
    ref = a * oracle.causal_conv(u1, f1, z0) + b * oracle.causal_conv(u1, f2, z0)
    assert _rel(y, ref) < 1e-13


def test_causal_conv_delta_shift_impulse():
    rng = np.random.default_rng(3)
    B, H, N = 2, 3, 128
    u = rng.standard_normal((B, H, N)); D = rng.standard_normal(H)
    # delta filter: y = (1 + D) u
    f = np.zeros((H, N)); f[:, 0] = 1.0
    y = oracle.causal_conv(u, f, D)
    np.testing.assert_allclose(y, (1.0 + D)[None, :, None] * u, rtol=1e-14, atol=0)
    # shifted delta: y_t = u_{t-s} (zeros before 0), no residual
    for s in (1, 7, N - 1):
        f = np.zeros((H, N)); f[:, s] = 1.0
        y = oracle.causal_conv(u, f, np.zeros(H))
        ref = np.zeros_like(u); ref[..., s:] = u[..., : N - s]
        assert np.array_equal(y, ref)
    # impulse input: y = f + D delta
    f = rng.standard_normal((H, N))
    ui = np.zeros((1, H, N)); ui[..., 0] = 1.0
    y = oracle.causal_conv(ui, f, D)
    ref = f.copy(); ref[:, 0] += D
    assert np.array_equal(y[0], ref)


# ---------------------------------------------------------------- SSM

def test_filter_conv_equals_recurrence():
    """Convolutional view == recurrent view (zero initial state), random SSMs."""
    rng = np.random.default_rng(4)
    B, H, S, N = 2, 3, 8, 300
    A, Bm, C, dt = _rand_ssm(rng, H, S)
    D = rng.standard_normal(H)
    u = rng.standard_normal((B, H, N))
    f = oracle.ssm_filter(A, Bm, C, dt, N)
    y_conv = oracle.causal_conv(u, f, D)
    y_rec = oracle.ssm_recurrence(u, A, Bm, C, dt, D)
    assert _rel(y_conv, y_rec) < 1e-12


def test_filter_conv_equals_recurrence_workload_construction():
    """Same equality on the workloads' diag-SSM construction (A_j=-0.5+i*pi*j, 64 modes)."""
    rng = np.random.default_rng(5)
    B, H, S, N = 1, 4, 64, 512
    A = np.tile(-0.5 + 1j * math.pi * np.arange(S), (H, 1))
    Bm = np.ones((H, S), dtype=complex)
    C = 0.5 * (rng.standard_normal((H, S)) + 1j * rng.standard_normal((H, S)))
    dt = np.array([1e-3, 1e-2, 5e-2, 1e-1])
    D = rng.standard_normal(H)
    u = rng.standard_normal((B, H, N))
    f = oracle.ssm_filter(A, Bm, C, dt, N)
    assert _rel(oracle.causal_conv(u, f, D), oracle.ssm_recurrence(u, A, Bm, C, dt, D)) < 1e-12


def test_filter_is_impulse_response():
    rng = np.random.default_rng(6)
    H, S, N = 3, 5, 100
    A, Bm, C, dt = _rand_ssm(rng, H, S)
    ui = np.zeros((1, H, N)); ui[..., 0] = 1.0
    y = oracle.ssm_recurrence(ui, A, Bm, C, dt, np.zeros(H))
    f = oracle.ssm_filter(A, Bm, C, dt, N)
    assert _rel(y[0], f) < 1e-13


def test_single_real_mode_matches_lfilter():
    """S=1, real A and C, B=1: y = lfilter([2 C dt], [1, -exp(dt A)], u) + D u."""
    rng = np.random.default_rng(7)
    N = 400
    a, c, dt, D = -0.7, 0.3, 0.05, 1.25
    u = rng.standard_normal(N)
    y = oracle.ssm_recurrence(u[None, None], np.array([[a + 0j]]), np.array([[1 + 0j]]),
                              np.array([[c + 0j]]), np.array([dt]), np.array([D]))[0, 0]
    ref = scipy.signal.lfilter([2 * c * dt], [1.0, -math.exp(dt * a)], u) + D * u
    assert _rel(y, ref) < 1e-13


def test_constant_input_closed_form():
    """u = 1: y_t = 2 Re(C dt B (1 - a^{t+1}) / (1 - a)) + D with a = exp(dt A)."""
    N = 257
    A = -0.3 + 2.1j; Bm = 0.8 - 0.4j; C = 0.6 + 0.2j; dt = 0.07; D = -0.4
    u = np.ones((1, 1, N))
    y = oracle.ssm_recurrence(u, np.array([[A]]), np.array([[Bm]]), np.array([[C]]),
                              np.array([dt]), np.array([D]))[0, 0]
    a = np.exp(dt * A)
    t = np.arange(N)
    ref = 2 * np.real(C * dt * Bm * (1 - a ** (t + 1)) / (1 - a)) + D
    assert _rel(y, ref) < 1e-13


def test_state_update_matrix_and_split():
    """Final state = M_ux u with columns Abar^{N-1-k} Bbar (summary page, App. C
    "State Passing"); and two calls joined through x_in/x_out equal one call."""
    rng = np.random.default_rng(8)
    B, H, S, N, M = 2, 3, 6, 240, 97
    A, Bm, C, dt = _rand_ssm(rng, H, S)
    D = rng.standard_normal(H)
    u = rng.standard_normal((B, H, N))
    y, x = oracle.ssm_recurrence(u, A, Bm, C, dt, D, return_state=True)
    abar = np.exp(dt[:, None] * A)            # [H,S]
    bbar = dt[:, None] * Bm
    k = np.arange(N)
    Mux = (abar[:, :, None] ** (N - 1 - k)[None, None, :]) * bbar[:, :, None]   # [H,S,N]
    x_ref = np.einsum("hsn,bhn->bhs", Mux, u)
    assert _rel(x, x_ref) < 1e-12
    y1, x1 = oracle.ssm_recurrence(u[..., :M], A, Bm, C, dt, D, return_state=True)
    y2, x2 = oracle.ssm_recurrence(u[..., M:], A, Bm, C, dt, D, x_in=x1, return_state=True)
    assert _rel(np.concatenate([y1, y2], axis=-1), y) < 1e-13
    assert _rel(x2, x) < 1e-13


def test_initial_state_term():
    """Zero input: y_t = 2 Re(sum_j C_j Abar_j^{t+1} x_in_j) (free response)."""
    rng = np.random.default_rng(9)
    H, S, N = 2, 4, 50
    A, Bm, C, dt = _rand_ssm(rng, H, S)
    x_in = rng.standard_normal((1, H, S)) + 1j * rng.standard_normal((1, H, S))
    y = oracle.ssm_recurrence(np.zeros((1, H, N)), A, Bm, C, dt, np.ones(H), x_in=x_in)
    abar = np.exp(dt[:, None] * A)
    t = np.arange(N)
    ref = 2 * np.real(np.einsum("hs,hst->ht", C * x_in[0], abar[:, :, None] ** (t + 1)[None, None]))
    assert _rel(y[0], ref) < 1e-12


# ---------------------------------------------------------------- H3 mix

def _h3_inputs(rng, B=2, N=96, Dm=5, L=4):
    q, k, v = rng.standard_normal((3, B, N, Dm))
    w = 0.5 * rng.standard_normal((Dm, L))
    f = rng.standard_normal((Dm, N)) * np.exp(-np.arange(N) / 16.0)
    D = rng.standard_normal(Dm)
    return q, k, v, w, f, D


def test_h3_mix_reduces_to_long_conv():
    """q = v = 1 and w = delta_0: out = causal_conv(k, f, D) (channel-last)."""
    rng = np.random.default_rng(10)
    q, k, v, w, f, D = _h3_inputs(rng)
    w = np.zeros_like(w); w[:, 0] = 1.0
    out = oracle.h3_mix(np.ones_like(q), k, np.ones_like(v), w, f, D)
    ref = oracle.causal_conv(np.transpose(k, (0, 2, 1)), f, D)
    assert _rel(np.transpose(out, (0, 2, 1)), ref) < 1e-14


def test_h3_mix_gates_only():
    """f = 0, D = 1: out = q * shift(k) * v, shift by numpy's convolution per channel."""
    rng = np.random.default_rng(11)
    q, k, v, w, f, D = _h3_inputs(rng)
    B, N, Dm = q.shape
    out = oracle.h3_mix(q, k, v, w, np.zeros_like(f), np.ones(Dm))
    s = np.empty_like(k)
    for b in range(B):
        for d in range(Dm):
            s[b, :, d] = np.convolve(k[b, :, d], w[d])[:N]
    assert _rel(out, q * s * v) < 1e-14


def test_h3_mix_single_tap():
    """L = 1, w = 1: out = q * causal_conv(k * v, f, D)."""
    rng = np.random.default_rng(12)
    q, k, v, _, f, D = _h3_inputs(rng)
    out = oracle.h3_mix(q, k, v, np.ones((q.shape[2], 1)), f, D)
    kv = np.transpose(k * v, (0, 2, 1))
    ref = np.transpose(oracle.causal_conv(kv, f, D), (0, 2, 1)) * q
    assert _rel(out, ref) < 1e-14


def test_h3_mix_shift_delay():
    """w = delta_1: the shift SSM is a one-step delay, s_t = k_{t-1}, s_0 = 0."""
    rng = np.random.default_rng(13)
    q, k, v, w, f, D = _h3_inputs(rng)
    w = np.zeros_like(w); w[:, 1] = 1.0
    out = oracle.h3_mix(q, k, v, w, np.zeros_like(f), np.ones(q.shape[2]))
    s = np.zeros_like(k); s[:, 1:, :] = k[:, :-1, :]
    assert np.array_equal(out, q * (s * v))


# ---------------------------------------------------------------- backward pass

def test_golden_causal_conv_bwd():
    g = _read_golden("causal_conv_bwd_hand.txt")
    f = g["f"][None, :]
    D = g["D"]
    # row 0 alone
    du, df, dD = oracle.causal_conv_bwd(g["u0"][None, None, :], f, D, g["dy0"][None, None, :])
    assert np.array_equal(du[0, 0], g["du0"])
    assert np.array_equal(df[0], g["df_row0"]) and np.array_equal(dD, g["dD_row0"])
    # both rows: du per row, df and dD summed over the batch
    u = np.stack([g["u0"], g["u1"]])[:, None, :]
    dy = np.stack([g["dy0"], g["dy1"]])[:, None, :]
    du, df, dD = oracle.causal_conv_bwd(u, f, D, dy)
    assert np.array_equal(du[0, 0], g["du0"]) and np.array_equal(du[1, 0], g["du1"])
    assert np.array_equal(df[0], g["df"]) and np.array_equal(dD, g["dD"])


@pytest.mark.parametrize("N", [1, 2, 7, 33, 64])
def test_causal_conv_bwd_bruteforce_exact(N):
    """Small integers: fp64 is exact, so compare bitwise with the transposed
    Jacobians built in integers (J_u = Toeplitz(f) + D I, J_f[t][s] = u[t-s])."""
    rng = np.random.default_rng(100 + N)
    B, H = 3, 2
    u = rng.integers(-6, 7, size=(B, H, N))
    dy = rng.integers(-6, 7, size=(B, H, N))
    f = rng.integers(-6, 7, size=(H, N))
    D = rng.integers(-3, 4, size=H)
    du, df, dD = oracle.causal_conv_bwd(u.astype(float), f.astype(float), D.astype(float), dy.astype(float))
    for h in range(H):
        fh, Dh = [int(x) for x in f[h]], int(D[h])
        df_ref = [0] * N
        dD_ref = 0
        for b in range(B):
            ub, dyb = [int(x) for x in u[b, h]], [int(x) for x in dy[b, h]]
            Ju = [[(fh[t - k] if k <= t else 0) + (Dh if k == t else 0) for k in range(N)] for t in range(N)]
            du_ref = [sum(Ju[t][k] * dyb[t] for t in range(N)) for k in range(N)]
            assert du[b, h].tolist() == [float(x) for x in du_ref]
            Jf = [[ub[t - s] if s <= t else 0 for s in range(N)] for t in range(N)]
            for s in range(N):
                df_ref[s] += sum(Jf[t][s] * dyb[t] for t in range(N))
            dD_ref += sum(dyb[t] * ub[t] for t in range(N))
        assert df[h].tolist() == [float(x) for x in df_ref]
        assert dD[h] == float(dD_ref)


def test_causal_conv_bwd_vs_numpy_convolve():
    """Library cross-check: du from a convolution of the reversed dy with f,
    df from a convolution of the reversed u with dy."""
    rng = np.random.default_rng(7)
    B, H, N = 2, 3, 257
    u, dy = rng.standard_normal((2, B, H, N))
    f = rng.standard_normal((H, N)); D = rng.standard_normal(H)
    du, df, dD = oracle.causal_conv_bwd(u, f, D, dy)
    for h in range(H):
        dfr = np.zeros(N)
        for b in range(B):
            ref = np.convolve(dy[b, h][::-1], f[h])[:N][::-1] + D[h] * dy[b, h]
            assert _rel(du[b, h], ref) < 1e-13
            dfr += np.convolve(u[b, h][::-1], dy[b, h])[N - 1:2 * N - 1]
        assert _rel(df[h], dfr) < 1e-13
        assert abs(dD[h] - np.sum(dy[:, h] * u[:, h])) < 1e-12 * np.sum(np.abs(dy[:, h] * u[:, h]))


def test_causal_conv_bwd_adjoint_of_the_forward():
    """The gradients are the adjoint of the oracle's own forward map:
    <dy, y(v, f, D)> = <du, v>,  <dy, y(u, g, 0)> = <df, g>,  and the D term."""
    rng = np.random.default_rng(8)
    B, H, N = 3, 2, 300
    u, dy, v = rng.standard_normal((3, B, H, N))
    f, g = rng.standard_normal((2, H, N))
    D, E = rng.standard_normal((2, H))
    du, df, dD = oracle.causal_conv_bwd(u, f, D, dy)
    lhs = np.sum(dy * oracle.causal_conv(v, f, D))
    assert abs(lhs - np.sum(du * v)) < 1e-11 * np.sum(np.abs(dy * oracle.causal_conv(v, f, D)))
    lhs = np.sum(dy * oracle.causal_conv(u, g, np.zeros(H)))
    assert abs(lhs - np.sum(df * g)) < 1e-11 * max(1.0, abs(lhs))
    lhs = np.sum(dy * oracle.causal_conv(u, np.zeros((H, N)), E))
    assert abs(lhs - np.sum(dD * E)) < 1e-11 * max(1.0, abs(lhs))


# ---------------------------------------------------------------- bidirectional copies

def test_golden_bidir_conv():
    g = _read_golden("causal_conv_hand.txt")
    y = oracle.bidir_conv(g["bidir_u"][None, None, :], g["bidir_f"][None, :], g["bidir_g"][None, :], g["bidir_D"])
    assert np.array_equal(y[0, 0], g["bidir_y"])


@pytest.mark.parametrize("N", [1, 3, 16, 50])
def test_bidir_conv_bruteforce_exact(N):
    """Small integers, exact in fp64: the full (upper + lower triangular)
    Toeplitz matrix built in integers."""
    rng = np.random.default_rng(300 + N)
    B, H = 2, 2
    u = rng.integers(-5, 6, size=(B, H, N)); f = rng.integers(-5, 6, size=(H, N))
    g = rng.integers(-5, 6, size=(H, N)); D = rng.integers(-3, 4, size=H)
    y = oracle.bidir_conv(u.astype(float), f.astype(float), g.astype(float), D.astype(float))
    for b in range(B):
        for h in range(H):
            T = [[(int(f[h, t - k]) if k <= t else 0) + (int(g[h, k - t]) if k >= t else 0) + (int(D[h]) if k == t else 0)
                  for k in range(N)] for t in range(N)]
            ref = [sum(T[t][k] * int(u[b, h, k]) for k in range(N)) for t in range(N)]
            assert y[b, h].tolist() == [float(x) for x in ref]


def test_bidir_conv_reductions():
    """g = 0 is the causal convolution; f = 0 is the causal convolution of the
    reversed input with g, reversed back (the anti-causal copy)."""
    rng = np.random.default_rng(31)
    B, H, N = 2, 3, 200
    u = rng.standard_normal((B, H, N)); f, g = rng.standard_normal((2, H, N)); D = rng.standard_normal(H)
    z = np.zeros((H, N))
    assert _rel(oracle.bidir_conv(u, f, z, D), oracle.causal_conv(u, f, D)) < 1e-14
    rev = oracle.causal_conv(u[..., ::-1].copy(), g, D)[..., ::-1]
    assert _rel(oracle.bidir_conv(u, z, g, D), rev) < 1e-13


# ---------------------------------------------------------------- multi-head H3

def test_golden_h3_mix_mh():
    g = _read_golden("h3_mix_hand.txt")
    q, k, v = (g["mh_" + x].reshape(1, 2, 2) for x in ("q", "k", "v"))
    w = g["mh_w"].reshape(2, 1)
    f = g["mh_f"].reshape(4, 2)
    out = oracle.h3_mix_mh(q, k, v, w, f, np.zeros(4), 2)
    assert np.array_equal(out.reshape(-1), g["mh_out"])


def test_h3_mix_mh_head_dim_one_is_h3_mix():
    rng = np.random.default_rng(41)
    B, N, Dm, L = 2, 90, 5, 3
    q, k, v = rng.standard_normal((3, B, N, Dm))
    w = rng.standard_normal((Dm, L)); f = rng.standard_normal((Dm, N)); D = rng.standard_normal(Dm)
    assert _rel(oracle.h3_mix_mh(q, k, v, w, f, D, 1), oracle.h3_mix(q, k, v, w, f, D)) < 1e-14


def test_h3_mix_mh_gates_only_closed_form():
    """f = 0, D = 1: out_j = (sum_i q_i s_i) v_j per head, s = shift(k)."""
    rng = np.random.default_rng(42)
    B, N, dh, heads, L = 2, 40, 4, 3, 2
    Dm = dh * heads
    q, k, v = rng.standard_normal((3, B, N, Dm))
    w = rng.standard_normal((Dm, L))
    out = oracle.h3_mix_mh(q, k, v, w, np.zeros((Dm * dh, N)), np.ones(Dm * dh), dh)
    s = w[None, None, :, 0] * k
    s[:, 1:, :] += w[None, None, :, 1] * k[:, :-1, :]
    qs = (q * s).reshape(B, N, heads, dh).sum(-1)                 # [B, N, heads]
    ref = (qs[..., None] * v.reshape(B, N, heads, dh)).reshape(B, N, Dm)
    assert _rel(out, ref) < 1e-13


def test_h3_mix_mh_entry_filters_are_separate():
    """A delta filter on one state entry (i, j) and zeros elsewhere routes
    exactly q_i s_i v_j to output channel j (catches swapped i, j)."""
    rng = np.random.default_rng(43)
    B, N, dh = 1, 30, 3
    q, k, v = rng.standard_normal((3, B, N, dh))
    w = np.ones((dh, 1))
    for i in range(dh):
        for j in range(dh):
            f = np.zeros((dh * dh, N)); f[i * dh + j, 0] = 1.0
            out = oracle.h3_mix_mh(q, k, v, w, f, np.zeros(dh * dh), dh)
            ref = np.zeros_like(out)
            ref[0, :, j] = q[0, :, i] * k[0, :, i] * v[0, :, j]
            assert _rel(out, ref) < 1e-15
