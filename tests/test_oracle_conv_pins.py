"""Pins for the oracle's causal depthwise convolution (oracle.causal_conv1d), the
front end that feeds the scan.

Tied to things other than itself: numpy.convolve of each row (the library routine
for a full discrete convolution, truncated to the causal part), the impulse
response (an input spike returns the reversed weights), scipy.special.expit for the
SiLU, causality, and the continuation rule (one call over [0, L) equals a call over
[0, s) followed by a call over [s, L) that starts from the first call's state).  A
flipped kernel, an off-by-one shift, a dropped bias or a wrong state order each fails
one of them.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_matches_numpy_convolve(K):
    x, w, b = rand((2, 5, 37), 1), rand((5, K), 2), rand(5, 3)
    out, _ = oracle.causal_conv1d(x, w, b, silu=False)
    for bb in range(2):
        for d in range(5):
            ref = np.convolve(x[bb, d], w[d, ::-1], mode="full")[:37] + b[d]
            np.testing.assert_allclose(out[bb, d], ref, rtol=1e-13, atol=1e-13)


def test_impulse_response_is_reversed_weights():
    K, L, t0 = 4, 12, 5
    w = np.array([[0.5, -1.25, 2.0, 3.5]])
    x = np.zeros((1, 1, L))
    x[0, 0, t0] = 1.0
    out, _ = oracle.causal_conv1d(x, w, silu=False)
    expect = np.zeros(L)
    expect[t0:t0 + K] = w[0, ::-1]
    np.testing.assert_array_equal(out[0, 0], expect)


def test_silu_is_applied_after_the_bias():
    x, w, b = rand((1, 3, 20), 4), rand((3, 4), 5), rand(3, 6)
    pre, _ = oracle.causal_conv1d(x, w, b, silu=False)
    out, _ = oracle.causal_conv1d(x, w, b, silu=True)
    np.testing.assert_allclose(out, pre * expit(pre), rtol=1e-14, atol=1e-15)


def test_causality():
    x, w = rand((1, 2, 30), 7), rand((2, 4), 8)
    base, _ = oracle.causal_conv1d(x, w)
    x2 = x.copy()
    x2[..., 17:] += 3.0
    out, _ = oracle.causal_conv1d(x2, w)
    np.testing.assert_array_equal(out[..., :17], base[..., :17])
    assert np.all(out[..., 17] != base[..., 17])


@pytest.mark.parametrize("K,s", [(4, 1), (4, 2), (4, 13), (3, 7), (2, 1), (1, 5)])
def test_split_with_state_continues_exactly(K, s):
    x, w, b = rand((2, 3, 25), 9), rand((3, K), 10), rand(3, 11)
    full, st_full = oracle.causal_conv1d(x, w, b)
    first, st = oracle.causal_conv1d(x[..., :s], w, b)
    second, st2 = oracle.causal_conv1d(x[..., s:], w, b, state=st if K > 1 else None)
    np.testing.assert_allclose(np.concatenate([first, second], axis=-1), full, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(st2, st_full, rtol=0, atol=0)
    # the state is the last K-1 inputs, oldest first
    np.testing.assert_array_equal(st_full, x[..., 25 - (K - 1):])


def test_short_sequence_state_mixes_history_and_input():
    K = 4
    x, w = rand((1, 1, 2), 12), rand((1, K), 13)
    hist = np.array([[[7.0, 8.0, 9.0]]])
    _, st = oracle.causal_conv1d(x, w, state=hist)
    np.testing.assert_array_equal(st, [[[9.0, x[0, 0, 0], x[0, 0, 1]]]])


def test_conv_refusals():
    with pytest.raises(oracle.OracleError):
        oracle.causal_conv1d(np.full((1, 1, 3), np.inf), np.ones((1, 2)))
    with pytest.raises(oracle.OracleError):
        oracle.causal_conv1d(np.ones((1, 1, 3)), np.ones((1, 9)))
