"""Pins of the convolution oracle (oracle/conv.py) against closed forms and
structural properties that do not restate its formula.  CPU only."""
import numpy as np

from oracle import conv as C


def _inputs(seed, L=5, H=12):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((L, H)), rng.standard_normal(H), rng.standard_normal((2 * H, H))


def test_identity_current_tap_squares():
    # current taps = x_t (identity generator), previous taps = 0: y = x * x
    x, x0, _ = _inputs(1)
    H = x.shape[1]
    Wt = np.vstack([np.eye(H), np.zeros((H, H))])
    np.testing.assert_array_equal(C.conv2tap(x, x0, Wt), x * x)


def test_identity_previous_tap_shifts():
    # previous taps = x_t: y_t = x_t * x_{t-1}, and the first position uses x0
    x, x0, _ = _inputs(2)
    H = x.shape[1]
    Wt = np.vstack([np.zeros((H, H)), np.eye(H)])
    y = C.conv2tap(x, x0, Wt)
    np.testing.assert_array_equal(y[0], x[0] * x0)
    np.testing.assert_array_equal(y[1:], x[1:] * x[:-1])


def test_permutation_generator_fixes_orientation():
    # Wt[c, k] = 1 iff k = (c + 1) mod H: the current tap of channel c is
    # x_t[(c + 1) mod H]; reading Wt transposed would give x_t[(c - 1) mod H]
    x, x0, _ = _inputs(3)
    H = x.shape[1]
    P = np.zeros((H, H))
    P[np.arange(H), (np.arange(H) + 1) % H] = 1.0
    Wt = np.vstack([P, np.zeros((H, H))])
    y = C.conv2tap(x, x0, Wt)
    np.testing.assert_array_equal(y, np.roll(x, -1, axis=1) * x)
    assert not np.allclose(y, np.roll(x, 1, axis=1) * x)


def test_quadratic_homogeneity():
    x, x0, Wt = _inputs(4)
    a = 1.75
    np.testing.assert_allclose(C.conv2tap(a * x, a * x0, Wt), a * a * C.conv2tap(x, x0, Wt), rtol=1e-12, atol=1e-12)


def test_linear_in_the_generator():
    x, x0, W1 = _inputs(5)
    W2 = np.random.default_rng(6).standard_normal(W1.shape)
    np.testing.assert_allclose(C.conv2tap(x, x0, W1 + W2), C.conv2tap(x, x0, W1) + C.conv2tap(x, x0, W2),
                               rtol=1e-12, atol=1e-12)


def test_causal_two_tap():
    # y_t depends on x_t and x_{t-1} only; x0 only reaches the first position
    x, x0, Wt = _inputs(7, L=6)
    y = C.conv2tap(x, x0, Wt)
    x2 = x.copy()
    x2[3] += 1.0
    y2 = C.conv2tap(x2, x0, Wt)
    np.testing.assert_array_equal(y2[:3], y[:3])
    np.testing.assert_array_equal(y2[5:], y[5:])
    assert not np.allclose(y2[3], y[3]) and not np.allclose(y2[4], y[4])
    y3 = C.conv2tap(x, x0 + 1.0, Wt)
    np.testing.assert_array_equal(y3[1:], y[1:])
    assert not np.allclose(y3[0], y[0])


def test_batch_is_independent_streams():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((3, 4, 8))
    x0 = rng.standard_normal((3, 8))
    Wt = rng.standard_normal((16, 8))
    yb = C.conv2tap_batch(x, x0, Wt)
    for b in range(3):
        np.testing.assert_array_equal(yb[b], C.conv2tap(x[b], x0[b], Wt))
