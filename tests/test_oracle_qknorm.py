"""Pins of the oracle's QK-norm ("SageBwd: A Trainable Low-bit Attention",
Methodology 4: query and key rows scaled to unit L2 norm before the dot
product): closed forms of the forward, a finite-difference check of the
backward against the unrounded map x -> x / |x| in fp64, and its invariants
(the gradient is orthogonal to x; scaling x by a power of two scales the
gradient by its inverse)."""
import numpy as np

import oracle as orc


def test_forward_closed_forms():
    X = np.zeros((4, 128), np.float32)
    X[0, 0] = 2.0                        # r = 1/2, y = e_0
    X[1, :] = 1.0                        # r = 2^-3.5, every y_c equal
    X[2, 0], X[2, 1] = 3.0, 4.0          # y = (0.6, 0.8) up to bf16 rounding
    # row 3: zero -> y = 0, r = 0
    Y, r = orc.qk_norm(X)
    assert r[0] == 0.5 and Y[0, 0] == 1.0 and np.all(Y[0, 1:] == 0.0)
    assert r[1] == np.float32(2.0 ** -3.5)
    assert np.all(Y[1] == Y[1, 0]) and abs(float(Y[1, 0]) - 2.0 ** -3.5) <= 2.0 ** -3.5 * 2.0 ** -8
    assert r[2] == np.float32(0.2)
    assert Y[2, 0] == 0.6015625 and Y[2, 1] == 0.80078125    # the bf16 neighbours of 0.6 and 0.8
    assert r[3] == 0.0 and np.all(Y[3] == 0.0)


def test_forward_is_unit_norm_within_bf16():
    rng = np.random.default_rng(3)
    X = (rng.standard_normal((64, 128)) * rng.uniform(0.01, 100.0, (64, 1))).astype(np.float32)
    Y, r = orc.qk_norm(X)
    n = np.linalg.norm(Y.astype(np.float64), axis=1)
    assert np.all(np.abs(n - 1.0) < 2.0 ** -8)
    np.testing.assert_allclose(r, 1.0 / np.linalg.norm(X.astype(np.float64), axis=1), rtol=2e-7)


def test_backward_closed_form():
    X = np.zeros((1, 2), np.float32)
    X[0] = (3.0, 4.0)
    _, r = orc.qk_norm(X)
    dX = orc.qk_norm_bwd(X, r, np.array([[1.0, 0.0]]))
    # r (g - y (y . g)) with r = 1/5, y = (0.6, 0.8): (0.128, -0.096), up to fp32(0.2)
    np.testing.assert_allclose(dX[0], [0.128, -0.096], rtol=1e-7)


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(9)
    d = 16
    X = rng.standard_normal((5, d)).astype(np.float32)
    G = rng.standard_normal((5, d))
    _, r = orc.qk_norm(X)
    dX = orc.qk_norm_bwd(X, r, G)
    f = lambda x: x / np.linalg.norm(x)
    eps = 1e-6
    for i in range(5):
        x = X[i].astype(np.float64)
        # the oracle uses fp32(1/|x|); the fp64 map's gradient differs from it by that rounding only
        num = np.array([(f(x + eps * e) - f(x - eps * e)) @ G[i] / (2 * eps) for e in np.eye(d)])
        np.testing.assert_allclose(dX[i], num, rtol=1e-6, atol=1e-8)
        assert abs(dX[i] @ x) < 1e-6 * np.linalg.norm(dX[i]) * np.linalg.norm(x)


def test_backward_scales_inversely():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((3, 128)).astype(np.float32)
    G = rng.standard_normal((3, 128))
    _, r = orc.qk_norm(X)
    _, r4 = orc.qk_norm(4.0 * X)
    np.testing.assert_array_equal(orc.qk_norm(4.0 * X)[0], orc.qk_norm(X)[0])
    np.testing.assert_allclose(orc.qk_norm_bwd(4.0 * X, r4, G), orc.qk_norm_bwd(X, r, G) / 4.0, rtol=1e-14)
