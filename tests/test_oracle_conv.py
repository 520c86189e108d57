"""Pins of the oracle's causal depthwise convolution (CPU): numpy's full convolution and scipy's
FIR filter (lfilter) per row, the state that continues a sequence, and the silu option."""
import numpy as np
import pytest
import scipy.signal

import oracle


@pytest.mark.parametrize("W", [1, 2, 4, 7])
def test_matches_numpy_and_scipy(W):
    rng = np.random.default_rng(W)
    Bt, Dc, L = 2, 3, 50
    x = rng.standard_normal((Bt, Dc, L))
    w = rng.standard_normal((Dc, W))
    bias = rng.standard_normal(Dc)
    out = oracle.conv1d(x, w, bias)
    for b in range(Bt):
        for d in range(Dc):
            # w[d, W-1] multiplies the newest input: the filter taps in time order are w[d, ::-1]
            want = np.convolve(x[b, d], w[d, ::-1])[:L] + bias[d]
            np.testing.assert_allclose(out[b, d], want, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(out[b, d], scipy.signal.lfilter(w[d, ::-1], [1.0], x[b, d]) + bias[d],
                                       rtol=1e-12, atol=1e-12)


def test_state_continues_the_sequence_and_silu():
    rng = np.random.default_rng(9)
    Bt, Dc, L, W, T = 1, 4, 40, 4, 13
    x = rng.standard_normal((Bt, Dc, L))
    w = rng.standard_normal((Dc, W))
    full = oracle.conv1d(x, w, silu=True)
    a, s = oracle.conv1d(x[..., :T], w, silu=True, return_state=True)
    np.testing.assert_array_equal(s, x[..., T - (W - 1):T])
    b = oracle.conv1d(x[..., T:], w, state=s, silu=True)
    np.testing.assert_allclose(np.concatenate([a, b], -1), full, rtol=1e-13, atol=1e-13)
    lin = oracle.conv1d(x, w)
    np.testing.assert_allclose(full, lin / (1.0 + np.exp(-lin)), rtol=1e-13, atol=1e-13)
