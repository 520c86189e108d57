"""Pins of the oracle's zero-order-hold option (CPU).

With zero-order hold the input coefficient is (exp(dt A) - 1) / A instead of dt (the explainer's
ZOH discretisation, sections 3 and 5).  Checked against scipy's own ZOH discretisation of the
continuous system (matrix exponential of the augmented system) simulated by scipy.signal.dlsim,
against the A -> 0 limit (dt, the Euler coefficient), and between the scalar-decay and diagonal
layouts.
"""
import numpy as np
import pytest
import scipy.signal

import oracle


@pytest.mark.parametrize("N,dt", [(1, 0.05), (4, 0.3), (6, 1.7)])
def test_matches_scipy_zoh_of_the_continuous_system(N, dt):
    rng = np.random.default_rng(N)
    L = 40
    A = -rng.uniform(0.2, 3.0, size=N)
    Bv, Cv = rng.standard_normal(N), rng.standard_normal(N)
    Dv = 0.7
    u = rng.standard_normal(L)
    sysd = scipy.signal.cont2discrete((np.diag(A), Bv[:, None], Cv[None, :], np.array([[Dv]])), dt, method="zoh")
    # scipy's discrete system outputs C h_{t-1} + D u_t (state before the update); the method's
    # readout is after the update, so compare against C (Ad h + Bd u) + D u
    Ad, Bd = sysd[0], sysd[1]
    h = np.zeros(N)
    want = np.empty(L)
    for t in range(L):
        h = Ad @ h + Bd[:, 0] * u[t]
        want[t] = Cv @ h + Dv * u[t]
    _, ys, xs = scipy.signal.dlsim(sysd, u[:, None])
    np.testing.assert_allclose(xs[1:], np.array([Ad @ xs[t] + Bd[:, 0] * u[t] for t in range(L - 1)]), atol=1e-12)
    got = oracle.scan_fwd(u[None, None, :], np.full((1, 1, L), dt), A[None, :], np.repeat(Bv[None, None, :, None], L, 3),
                          np.repeat(Cv[None, None, :, None], L, 3), np.array([Dv]), softplus=False, zoh=True)
    np.testing.assert_allclose(got[0, 0], want, rtol=1e-10, atol=1e-12)
    # and scipy's own outputs, shifted by its readout convention: y_scipy[t] = C h_{t-1} + D u_t
    np.testing.assert_allclose(ys[1:, 0] - Dv * u[1:], (got[0, 0] - Dv * u)[:-1], rtol=1e-10, atol=1e-12)


def test_small_decay_limit_is_the_euler_coefficient():
    rng = np.random.default_rng(3)
    Bt, Dc, L, N = 1, 3, 30, 4
    u, B, C = rng.standard_normal((Bt, Dc, L)), rng.standard_normal((Bt, 1, N, L)), rng.standard_normal((Bt, 1, N, L))
    delta = rng.uniform(0.01, 0.5, size=(Bt, Dc, L))
    A = np.full((Dc, N), -1e-9)
    zoh = oracle.scan_fwd(u, delta, A, B, C, softplus=False, zoh=True)
    euler = oracle.scan_fwd(u, delta, A, B, C, softplus=False, zoh=False)
    np.testing.assert_allclose(zoh, euler, rtol=1e-8, atol=1e-10)
    # and with a real decay the two differ (the option is not a no-op)
    A2 = -rng.uniform(0.5, 2.0, size=(Dc, N))
    assert np.max(np.abs(oracle.scan_fwd(u, delta, A2, B, C, softplus=False, zoh=True)
                         - oracle.scan_fwd(u, delta, A2, B, C, softplus=False, zoh=False))) > 1e-3


def test_scalar_decay_equals_diagonal_broadcast_with_zoh():
    rng = np.random.default_rng(4)
    Bt, H, P, L, N = 2, 2, 3, 25, 5
    Dc = H * P
    u, B, C = rng.standard_normal((Bt, Dc, L)), rng.standard_normal((Bt, 1, N, L)), rng.standard_normal((Bt, 1, N, L))
    delta = rng.standard_normal((Bt, H, L))
    Ah = -rng.uniform(0.3, 2.0, size=H)
    scalar = oracle.scan_fwd(u, delta, Ah, B, C, softplus=True, zoh=True)
    diag = oracle.scan_fwd(u, np.repeat(delta, P, axis=1), np.repeat(Ah, P)[:, None] * np.ones((1, N)), B, C,
                           softplus=True, zoh=True)
    np.testing.assert_allclose(scalar, diag, rtol=1e-12, atol=1e-12)
