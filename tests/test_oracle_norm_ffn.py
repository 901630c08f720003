"""Pins for the oracle's LayerNorm (no affine) and ReLU^2 x Mul backward: hand-worked
values, central differences of the forwards, and the invariants the formulas fix."""

import numpy as np
import pytest
import torch

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


# ----------------------------------------------------------------------------- FFN block

def _tiny_ffn(seed, T=3, C=6, F=5, kink_free=True):
    rng = np.random.default_rng(seed)
    p = dict(x=rng.standard_normal((T, C)), gamma1=rng.uniform(0.5, 1.5, C),
             w_gu=rng.standard_normal((C, 2 * F)) * 0.5, gamma2=rng.uniform(0.5, 1.5, F),
             w_down=rng.standard_normal((F, C)) * 0.5)
    if kink_free:   # keep every gate away from ReLU's kink so central differences apply
        _, sv = NF.ffn_forward(**p)
        assert np.min(np.abs(sv["gu"][:, :F])) > 1e-3
    return p


def _ffn_out(p, **over):
    q = dict(p, **over)
    return NF.ffn_forward(q["x"], q["gamma1"], q["w_gu"], q["gamma2"], q["w_down"])[0]


def test_ffn_backward_matches_central_differences():
    p = _tiny_ffn(11)
    dout = np.random.default_rng(12).standard_normal(p["x"].shape)
    _, sv = NF.ffn_forward(**p)
    dx, dwgu, dwd = NF.ffn_backward(sv, dout)
    for name, got in (("x", dx), ("w_gu", dwgu), ("w_down", dwd)):
        num = verify.numerical_grad(lambda z: float(np.sum(dout * _ffn_out(p, **{name: z}))), p[name], eps=1e-6)
        np.testing.assert_allclose(got, num, rtol=1e-6, atol=1e-7, err_msg=name)


def test_ffn_backward_matches_torch_autograd():
    # an independent statement of the same forward in torch float64 ops
    p = _tiny_ffn(13, T=4, C=8, F=6)
    dout = np.random.default_rng(14).standard_normal(p["x"].shape)
    _, sv = NF.ffn_forward(**p)
    dx, dwgu, dwd = NF.ffn_backward(sv, dout)
    t = {k: torch.tensor(v, requires_grad=k in ("x", "w_gu", "w_down")) for k, v in p.items()}

    def rms(z, g):
        return z * g / torch.sqrt((z * z).mean(dim=1, keepdim=True) + 1e-6)

    gu = rms(t["x"], t["gamma1"]) @ t["w_gu"]
    F = gu.shape[1] // 2
    h = torch.relu(gu[:, :F]) ** 2 * gu[:, F:]
    out = t["x"] + rms(h, t["gamma2"]) @ t["w_down"]
    (out * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(dx, t["x"].grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dwgu, t["w_gu"].grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dwd, t["w_down"].grad.numpy(), rtol=1e-12, atol=1e-13)


def test_ffn_backward_all_gates_closed_is_the_residual():
    # every gate <= 0: h = 0, so hn = 0 and the ReLU passes no gradient: dx = dout exactly,
    # and both weight gradients vanish
    p = _tiny_ffn(15, kink_free=False)
    p["w_gu"][:, :5] = -np.abs(p["w_gu"][:, :5])
    p["x"] = np.abs(p["x"])
    _, sv = NF.ffn_forward(**p)
    assert np.all(sv["gu"][:, :5] <= 0)
    dout = np.random.default_rng(16).standard_normal(p["x"].shape)
    dx, dwgu, dwd = NF.ffn_backward(sv, dout)
    np.testing.assert_array_equal(dx, dout)
    np.testing.assert_array_equal(dwgu, 0.0)
    np.testing.assert_array_equal(dwd, 0.0)


def test_ffn_planted_mistakes_fail_the_difference_check(monkeypatch):
    # plausible slips in the oracle's FFN backward must each break agreement with central
    # differences: dUp and dGate swapped, no residual, sub-norm backward skipped
    p = _tiny_ffn(17)
    dout = np.random.default_rng(18).standard_normal(p["x"].shape)
    _, sv = NF.ffn_forward(**p)
    num = verify.numerical_grad(lambda z: float(np.sum(dout * _ffn_out(p, x=z))), p["x"], eps=1e-6)
    good = NF.ffn_backward(sv, dout)[0]
    assert np.max(np.abs(good - num)) < 1e-6
    real = NF.relu2_mul_backward
    monkeypatch.setattr(NF, "relu2_mul_backward", lambda g, u, d: real(g, u, d)[::-1])
    assert np.max(np.abs(NF.ffn_backward(sv, dout)[0] - num)) > 1e-3
    monkeypatch.setattr(NF, "relu2_mul_backward", real)
    assert np.max(np.abs((NF.ffn_backward(sv, dout)[0] - dout) - num)) > 1e-3
    monkeypatch.setattr(NF, "rmsnorm_backward_rows", lambda x, g, dy, eps=1e-6: np.asarray(dy, np.float64))
    assert np.max(np.abs(NF.ffn_backward(sv, dout)[0] - num)) > 1e-3
