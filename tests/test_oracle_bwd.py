"""Pins of the oracle's backward (CPU): every gradient equals central finite differences of the
oracle's forward, sum(dy * y), on tiny float64 problems.  The finite differences use only the
forward definition, so they check the hand-derived reverse pass independently (a dropped term, a
wrong sign or a shifted step index in it changes some derivative by far more than the bar).
"""
import numpy as np
import pytest

import oracle


def problem(seed, Bt, Dc, L, N, H, G, scalar, gate, softplus, with_D=True, with_bias=True):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s)
    p = dict(u=f(Bt, Dc, L), B=f(Bt, G, N, L), C=f(Bt, G, N, L), z=f(Bt, Dc, L) if gate else None,
             A=-rng.uniform(0.3, 1.5, size=(H,) if scalar else (Dc, N)),
             D=f(H if (scalar and H != Dc) else Dc) if with_D else None)
    if softplus:
        p["delta"] = f(Bt, H, L)
        p["delta_bias"] = rng.uniform(-2.0, 0.5, size=H) if with_bias else None
    else:
        p["delta"] = rng.uniform(0.05, 0.6, size=(Bt, H, L))
        p["delta_bias"] = rng.uniform(0.0, 0.2, size=H) if with_bias else None
    return p


def loss(p, dy, softplus, h0):
    y = oracle.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"],
                        softplus=softplus, h0=h0, threads=1)
    return float(np.sum(dy * y))


CASES = [
    # seed, Bt, Dc, L, N, heads, groups, scalar decay, gate, softplus
    (1, 1, 4, 6, 3, 4, 2, False, True, True),
    (2, 2, 4, 5, 2, 2, 1, True, False, False),
    (3, 1, 6, 7, 4, 3, 3, True, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "seed%d" % c[0])
@pytest.mark.parametrize("with_h0", [False, True])
def test_gradients_match_finite_differences(case, with_h0):
    seed, Bt, Dc, L, N, H, G, scalar, gate, softplus = case
    p = problem(seed, Bt, Dc, L, N, H, G, scalar, gate, softplus)
    rng = np.random.default_rng(100 + seed)
    dy = rng.standard_normal((Bt, Dc, L))
    h0 = rng.standard_normal((Bt * Dc, N)) if with_h0 else None
    g = oracle.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"], dy=dy,
                        softplus=softplus, h0=h0, threads=2)
    names = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
             "delta_bias": "ddelta_bias"}
    checked = 0
    for key, gname in names.items():
        if p[key] is None:
            assert g[gname] is None
            continue
        x = p[key]
        fd = np.empty(x.shape)
        for idx in np.ndindex(x.shape):
            eps = 1e-6 * max(1.0, abs(x[idx]))
            old = x[idx]
            x[idx] = old + eps
            fp = loss(p, dy, softplus, h0)
            x[idx] = old - eps
            fm = loss(p, dy, softplus, h0)
            x[idx] = old
            fd[idx] = (fp - fm) / (2 * eps)
        err = np.max(np.abs(fd - g[gname]) / (1.0 + np.abs(fd)))
        assert err < 1e-6, (key, err)
        checked += x.size
    if with_h0:
        fd = np.empty(h0.shape)
        for idx in np.ndindex(h0.shape):
            old = h0[idx]
            h0[idx] = old + 1e-6
            fp = loss(p, dy, softplus, h0)
            h0[idx] = old - 1e-6
            fm = loss(p, dy, softplus, h0)
            h0[idx] = old
            fd[idx] = (fp - fm) / 2e-6
        assert np.max(np.abs(fd - g["dh0"]) / (1.0 + np.abs(fd))) < 1e-6
    assert checked > 50


def test_gradients_are_zero_without_upstream_gradient():
    p = problem(4, 1, 4, 5, 3, 4, 1, False, True, True)
    g = oracle.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"],
                        dy=np.zeros((1, 4, 5)), softplus=True)
    for k, v in g.items():
        if v is not None:
            assert not np.any(v), k


def test_rows_sum_into_shared_gradients():
    """dB, dC (shared by the channels of a group) and dA (shared by the batch) are sums over
    rows: the gradient of a two-channel problem is the sum of the one-channel gradients."""
    p = problem(5, 1, 2, 6, 3, 2, 1, False, False, True)
    dy = np.random.default_rng(6).standard_normal((1, 2, 6))
    full = oracle.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], None, p["delta_bias"], dy=dy)
    parts = []
    for d in range(2):
        q = dict(u=p["u"][:, d:d + 1], delta=p["delta"][:, d:d + 1], A=p["A"][d:d + 1], D=p["D"][d:d + 1],
                 delta_bias=p["delta_bias"][d:d + 1])
        parts.append(oracle.scan_bwd(q["u"], q["delta"], q["A"], p["B"], p["C"], q["D"], None, q["delta_bias"],
                                     dy=dy[:, d:d + 1]))
    np.testing.assert_allclose(full["dB"], parts[0]["dB"] + parts[1]["dB"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(full["dC"], parts[0]["dC"] + parts[1]["dC"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(full["dA"], np.concatenate([parts[0]["dA"], parts[1]["dA"]]), rtol=1e-13)
