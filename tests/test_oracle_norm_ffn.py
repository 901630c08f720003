"""Pins for the oracle's LayerNorm (no affine) and ReLU^2 x Mul backward: hand-worked
values, central differences of the forwards, and the invariants the formulas fix."""

import numpy as np
import pytest

from oracle import norm_ffn as NF
from oracle import verify


def test_layernorm_forward_hand_values():
    # x = (1, 2, 3, 6): mu 3, variance (4 + 1 + 0 + 9) / 4 = 3.5, sigma = sqrt(3.5 + 1e-5)
    y, sig = NF.layernorm_forward(np.array([[1.0, 2.0, 3.0, 6.0]]))
    s = np.sqrt(3.5 + 1e-5)
    assert sig[0] == pytest.approx(s, rel=1e-15)
    np.testing.assert_allclose(y[0], np.array([-2.0, -1.0, 0.0, 3.0]) / s, rtol=1e-15)


def test_layernorm_backward_hand_values():
    # y = (-1, 1), sigma = 2, dy = (3, 5): mean(dy) = 4, mean(dy y) = 1,
    # dx = ((3 - 4 + 1) / 2, (5 - 4 - 1) / 2) = (0, 0); dy = (1, 0): mean 0.5, mean(dy y) = -0.5,
    # dx = ((1 - 0.5 - 0.5) / 2, (0 - 0.5 + 0.5) / 2) = (0, 0); dy = (2, -2): dx = ((2 - 0 - 2) / 2, ...) = 0
    y, sig = np.array([[-1.0, 1.0]]), np.array([2.0])
    for dy in ([3.0, 5.0], [1.0, 0.0], [2.0, -2.0]):
        np.testing.assert_allclose(NF.layernorm_backward(np.array([dy]), y, sig), 0.0, atol=1e-15)
    # a width-3 row: y = (-1, 0, 1), sigma = 0.5, dy = (0, 1, 0): mean 1/3, mean(dy y) = 0
    dx = NF.layernorm_backward(np.array([[0.0, 1.0, 0.0]]), np.array([[-1.0, 0.0, 1.0]]), np.array([0.5]))
    np.testing.assert_allclose(dx[0], np.array([-1 / 3, 2 / 3, -1 / 3]) / 0.5, rtol=1e-15)


@pytest.mark.parametrize("C", [2, 7, 64])
def test_layernorm_backward_matches_central_differences(C):
    rng = np.random.default_rng(C)
    x = rng.standard_normal((3, C)) * 2.0 + 0.5
    dy = rng.standard_normal((3, C))
    y, sig = NF.layernorm_forward(x)
    num = verify.numerical_grad(lambda z: float(np.sum(dy * NF.layernorm_forward(z)[0])), x, eps=1e-6)
    np.testing.assert_allclose(NF.layernorm_backward(dy, y, sig), num, rtol=1e-7, atol=1e-8)


def test_layernorm_backward_invariants():
    # sum_j dx_j = 0 per row (y has zero mean), and a constant dy shifts nothing: dx = 0
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 33))
    y, sig = NF.layernorm_forward(x)
    dx = NF.layernorm_backward(rng.standard_normal((5, 33)), y, sig)
    np.testing.assert_allclose(dx.sum(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(NF.layernorm_backward(np.full((5, 33), 1.7), y, sig), 0.0, atol=1e-13)


def test_relu2_mul_hand_values():
    # gate 3, up 2, dh 0.5: h = 18, dGate = 0.5 * 2 * 2 * 3 = 6, dUp = 0.5 * 9 = 4.5;
    # gate -1: h = 0 and both gradients 0; gate 0: both 0
    g, u, d = np.array([3.0, -1.0, 0.0]), np.array([2.0, 5.0, 4.0]), np.array([0.5, 1.0, 1.0])
    np.testing.assert_array_equal(NF.relu2_mul_forward(g, u), [18.0, 0.0, 0.0])
    dg, du = NF.relu2_mul_backward(g, u, d)
    np.testing.assert_array_equal(dg, [6.0, 0.0, 0.0])
    np.testing.assert_array_equal(du, [4.5, 0.0, 0.0])


def test_relu2_mul_matches_central_differences():
    # the pages' check for this op (numerical gradient); points kept away from the kink at 0
    rng = np.random.default_rng(4)
    g = rng.standard_normal(40)
    g = np.where(np.abs(g) < 0.05, 0.3, g)
    u, dh = rng.standard_normal(40), rng.standard_normal(40)
    dg, du = NF.relu2_mul_backward(g, u, dh)
    ng = verify.numerical_grad(lambda z: float(np.sum(dh * NF.relu2_mul_forward(z, u))), g, eps=1e-6)
    nu = verify.numerical_grad(lambda z: float(np.sum(dh * NF.relu2_mul_forward(g, z))), u, eps=1e-6)
    np.testing.assert_allclose(dg, ng, rtol=1e-7, atol=1e-8)
    np.testing.assert_allclose(du, nu, rtol=1e-7, atol=1e-8)
