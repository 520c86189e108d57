"""Pins of the oracle's exponential-trapezoidal option (CPU).

The rule h_t = a_t h_{t-1} + 1/2 (e_t + a_t e_{t-1}) (the explainer's Mamba-3 recurrence,
section 6.3) integrates the input term of the continuous system by the trapezoid rule, so on a
smooth input its error against the exact continuous solution falls by ~4 when the step halves
(exponential-Euler: by ~2).  That and the exact solution (scipy's ODE solver) pin the rule
independently of how the oracle writes it; two further checks tie it to the Euler oracle and to
composition across a split of the sequence.
"""
import numpy as np
import pytest
from scipy.integrate import solve_ivp

import oracle


def exact_outputs(A, Bv, Cv, times, ufun):
    """y(t) = C h(t) of dh/dt = A h + B u(t), h(0) = 0, for diagonal A, by a tight ODE solve."""
    sol = solve_ivp(lambda t, h: A * h + Bv * ufun(t), (0.0, times[-1]), np.zeros(A.size), t_eval=times,
                    rtol=1e-12, atol=1e-14, method="DOP853")
    return Cv @ sol.y


def discrete_outputs(A, Bv, Cv, dt, L, ufun, trapezoid):
    t = dt * np.arange(1, L + 1)   # step t ends at time (t + 1) dt; its input is u there
    u = ufun(t)
    y = oracle.scan_fwd(u[None, None, :], np.full((1, 1, L), dt), A[None, :],
                        np.repeat(Bv[None, None, :, None], L, 3), np.repeat(Cv[None, None, :, None], L, 3),
                        softplus=False, trapezoid=trapezoid)
    return t, y[0, 0]


def test_second_order_against_the_continuous_system():
    rng = np.random.default_rng(1)
    N = 4
    A = -rng.uniform(0.5, 3.0, size=N)
    Bv, Cv = rng.standard_normal(N), rng.standard_normal(N)
    ufun = lambda t: np.sin(3.0 * t) + 0.5 * np.sin(7.0 * t)   # smooth, u(0) = 0
    errs = {}
    for trap in (False, True):
        e = []
        for dt in (0.02, 0.01, 0.005):
            L = int(round(2.0 / dt))
            t, y = discrete_outputs(A, Bv, Cv, dt, L, ufun, trap)
            e.append(np.max(np.abs(y - exact_outputs(A, Bv, Cv, t, ufun))))
        errs[trap] = e
    euler, trap = errs[False], errs[True]
    assert 1.7 < euler[0] / euler[1] < 2.3 and 1.7 < euler[1] / euler[2] < 2.3, euler
    assert 3.5 < trap[0] / trap[1] < 4.5 and 3.5 < trap[1] / trap[2] < 4.5, trap
    assert trap[-1] < 0.05 * euler[-1]


@pytest.mark.parametrize("scalar", [False, True])
def test_relation_to_the_euler_scan(scalar):
    """With e_t = dt B_t u_t, k_t = h_t + e_t / 2 obeys the Euler recurrence, so the trapezoidal
    output is the Euler output minus dt_t u_t (C_t . B_t) / 2 (before the gate)."""
    rng = np.random.default_rng(2)
    Bt, Dc, L, N, H = 2, 4, 30, 5, 2 if scalar else 4
    u = rng.standard_normal((Bt, Dc, L))
    delta = rng.standard_normal((Bt, H, L))
    A = -rng.uniform(0.3, 2.0, size=(H,) if scalar else (Dc, N))
    B, C = rng.standard_normal((Bt, 1, N, L)), rng.standard_normal((Bt, 1, N, L))
    D = rng.standard_normal(Dc)
    bias = rng.uniform(-2, 0, size=H)
    tr = oracle.scan_fwd(u, delta, A, B, C, D, None, bias, softplus=True, trapezoid=True)
    eu = oracle.scan_fwd(u, delta, A, B, C, D, None, bias, softplus=True)
    x = delta + bias[None, :, None]
    dt = np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))
    dt = np.repeat(dt, Dc // H, axis=1)
    cb = np.einsum("bnt,bnt->bt", C[:, 0], B[:, 0])[:, None, :]
    np.testing.assert_allclose(tr, eu - 0.5 * dt * u * cb, rtol=1e-11, atol=1e-11)


def test_pieces_compose_through_the_carried_state():
    rng = np.random.default_rng(3)
    Bt, Dc, L, N, T = 1, 3, 40, 4, 17
    u, delta = rng.standard_normal((Bt, Dc, L)), rng.standard_normal((Bt, Dc, L))
    A = -rng.uniform(0.3, 2.0, size=(Dc, N))
    B, C = rng.standard_normal((Bt, 1, N, L)), rng.standard_normal((Bt, 1, N, L))
    z = rng.standard_normal((Bt, Dc, L))
    kw = dict(softplus=True, trapezoid=True)
    full, hf = oracle.scan_fwd(u, delta, A, B, C, None, z, None, return_state=True, **kw)
    y1, h1 = oracle.scan_fwd(u[..., :T], delta[..., :T], A, B[..., :T], C[..., :T], None, z[..., :T], None,
                             return_state=True, **kw)
    y2, h2 = oracle.scan_fwd(u[..., T:], delta[..., T:], A, B[..., T:], C[..., T:], None, z[..., T:], None,
                             h0=h1, return_state=True, **kw)
    np.testing.assert_allclose(np.concatenate([y1, y2], -1), full, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h2, hf, rtol=1e-12, atol=1e-12)
