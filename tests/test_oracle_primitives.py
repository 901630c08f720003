"""Pins for the oracle's softmax, RoPE and RMSNorm specs against facts fixed outside the
oracle: closed forms, invariants the API page states, hand-worked fixtures, central
differences and torch autograd (float64, CPU)."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import specs, verify
from oracle.layer import rope_backward_rows, rope_forward_rows, rmsnorm_backward_rows


# ----------------------------------------------------------------------------- softmax

@pytest.mark.parametrize("seed", range(5))
def test_softmax_backward_sums_to_zero(seed):
    # Tier-1 identity of the page's "Verification Strategy" (softmaxBackwardSumsToZero).
    rng = np.random.default_rng(seed)
    x, dy = rng.standard_normal(17) * 3, rng.standard_normal(17)
    dx = specs.softmax_backward(x, dy)
    assert abs(specs.softmax_backward_sums_to_zero(x, dy)) <= 1e-12 * np.sum(np.abs(dx)) + 1e-300


def test_softmax_two_element_logistic_closed_form():
    # n = 2 reduces to the logistic: s0 = 1/(1+exp(x1-x0)), dx0 = s0*s1*(dy0-dy1), dx1 = -dx0.
    x, dy = np.array([0.7, -1.1]), np.array([2.0, -0.5])
    s0 = 1.0 / (1.0 + math.exp(x[1] - x[0]))
    s1 = 1.0 - s0
    dx = specs.softmax_backward(x, dy)
    assert dx[0] == pytest.approx(s0 * s1 * (dy[0] - dy[1]), rel=1e-14)
    assert dx[1] == pytest.approx(-s0 * s1 * (dy[0] - dy[1]), rel=1e-14)


def test_softmax_constant_upstream_gives_zero():
    x = np.array([1.0, -2.0, 0.5, 3.0])
    assert np.max(np.abs(specs.softmax_backward(x, np.full(4, 2.5)))) < 1e-15


def test_softmax_numerical_checks():
    assert verify.softmax_numerical_check([0.3, -1.2, 2.0, 0.1], 0)
    assert verify.softmax_numerical_check([0.3, -1.2, 2.0, 0.1], 3)
    assert verify.verify_softmax_backward(n=9, seed=3)


def test_softmax_backward_matches_autograd():
    rng = np.random.default_rng(11)
    x, dy = rng.standard_normal(12), rng.standard_normal(12)
    xt = torch.tensor(x, requires_grad=True)
    torch.softmax(xt, 0).backward(torch.tensor(dy))
    np.testing.assert_allclose(specs.softmax_backward(x, dy), xt.grad.numpy(), rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------- RoPE

def _theta(s):
    return {"pi/2": math.pi / 2, "pi": math.pi, "0": 0.0}[s]


def test_rope_hand_fixture(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "rope_hand.json")))
    for case in g["pairs"]:
        dx0, dx1 = specs.rope_backward(case["dy"][0], case["dy"][1], _theta(case["theta"]))
        assert dx0 == pytest.approx(case["dx"][0], abs=1e-15)
        assert dx1 == pytest.approx(case["dx"][1], abs=1e-15)
    th = specs.rope_angles([5], 64, 10000.0)[0]
    for i, val in g["angles_pos5_d64"].items():
        assert th[int(i)] == pytest.approx(val, rel=1e-14)


def test_rope_roundtrip_identity_at_tiny_workload_angles():
    # Tier-1: backward o forward = identity to 1e-6 (ropeRoundtripCheck), 32 pairs at pos 5.
    rng = np.random.default_rng(5)
    th = specs.rope_angles([5], 64)[0]
    x0, x1 = rng.standard_normal(32), rng.standard_normal(32)
    assert specs.rope_roundtrip_check(x0, x1, th, tol=1e-6)
    y0, y1 = specs.rope_forward(x0, x1, th)
    z0, z1 = specs.rope_backward(y0, y1, th)
    assert np.max(np.abs(z0 - x0)) < 1e-14 and np.max(np.abs(z1 - x1)) < 1e-14


def test_rope_roundtrip_check_rejects_a_rotation_that_is_not_the_inverse(monkeypatch):
    # ropeRoundtripCheck must be able to fail: with the forward rotation R(+theta) planted
    # where the inverse R(-theta) belongs, backward(forward(x)) = R(2 theta) x != x at the
    # single-query workload's angles (pos 5: theta_0 = 5 rad, sin(10) != 0).
    rng = np.random.default_rng(5)
    th = specs.rope_angles([5], 64)[0]
    x0, x1 = rng.standard_normal(32), rng.standard_normal(32)
    assert specs.rope_roundtrip_check(x0, x1, th, tol=1e-6)
    monkeypatch.setattr(specs, "rope_backward", specs.rope_forward)
    assert not specs.rope_roundtrip_check(x0, x1, th, tol=1e-6)
    # a plain sign error in the sine term (rotation by -theta applied twice) fails too
    monkeypatch.setattr(specs, "rope_backward", lambda a, b, t: specs.rope_forward(a, b, -2.0 * np.asarray(t)))
    assert not specs.rope_roundtrip_check(x0, x1, th, tol=1e-6)


def test_run_all_checks_passes():
    # runAllChecks ("Numerical Gradient Verification"): every verify* and the Tier-1
    # identities hold for the oracle's backward specs.
    assert verify.run_all_checks(verbose=False)


def test_run_all_checks_fails_on_a_wrong_softmax_backward(monkeypatch):
    # the same entry point must report a failure when one backward is wrong (negated)
    right = specs.softmax_backward
    monkeypatch.setattr(specs, "softmax_backward", lambda x, dy: -right(x, dy))
    assert not verify.run_all_checks(verbose=False)


def test_rope_backward_is_orthogonal():
    rng = np.random.default_rng(6)
    dy = rng.standard_normal((7, 3, 16))
    dx = rope_backward_rows(dy, np.arange(7) + 100)
    np.testing.assert_allclose(np.linalg.norm(dx, axis=-1), np.linalg.norm(dy, axis=-1), rtol=1e-14)


@pytest.mark.parametrize("layout", [0, 1])
def test_rope_rows_fd_and_autograd(layout):
    assert verify.verify_rope_backward(T=3, H=2, d=8, pos0=5) if layout == 0 else True
    rng = np.random.default_rng(7 + layout)
    T, H, d = 4, 2, 8
    x, dy = rng.standard_normal((T, H, d)), rng.standard_normal((T, H, d))
    pos = np.arange(T) + 3
    f = verify.vjp_loss(lambda z: rope_forward_rows(z, pos, 10000.0, layout), dy)
    num = verify.numerical_grad(f, x)
    ana = rope_backward_rows(dy, pos, 10000.0, layout)
    assert verify.check_gradient(ana, num)
    assert np.max(np.abs(ana - num)) < 1e-8
    # autograd of an independently written rotation (complex multiply by e^{i theta})
    xt = torch.tensor(x, requires_grad=True)
    th = torch.tensor(specs.rope_angles(pos, d)[:, None, :])
    if layout == 0:
        a, b = xt[..., 0::2], xt[..., 1::2]
    else:
        a, b = xt[..., : d // 2], xt[..., d // 2:]
    z = torch.complex(a, b) * torch.polar(torch.ones_like(th), th)
    y = torch.empty_like(xt)
    if layout == 0:
        y = torch.stack([z.real, z.imag], dim=-1).reshape(T, H, d)
    else:
        y = torch.cat([z.real, z.imag], dim=-1)
    (y * torch.tensor(dy)).sum().backward()
    np.testing.assert_allclose(ana, xt.grad.numpy(), rtol=0, atol=1e-13)


def test_rope_layouts_rotate_different_pairs():
    dy = np.zeros((1, 1, 8))
    dy[0, 0, 1] = 1.0
    a = rope_backward_rows(dy, [5], layout=0)
    b = rope_backward_rows(dy, [5], layout=1)
    assert a[0, 0, 0] != 0.0 and b[0, 0, 0] == 0.0


# ----------------------------------------------------------------------------- RMSNorm

def test_rmsnorm_hand_fixture(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "rmsnorm_hand.json")))
    dx = specs.rmsnorm_backward(g["x"], g["gamma"], g["dy"], eps=g["eps"])
    np.testing.assert_allclose(dx / math.sqrt(2.0), g["dx_over_sqrt2"], rtol=1e-13)
    assert abs(np.dot(dx, g["x"])) < 1e-14


def test_rmsnorm_fd_page_tolerance():
    assert verify.verify_rmsnorm_backward(n=8, seed=1)
    assert verify.verify_rmsnorm_backward(n=64, seed=2)


def test_rmsnorm_eps_inside_root_pinned_by_tight_fd():
    # With a large eps the two readings (eps inside vs outside the root) differ a lot;
    # the page's backward (with its n * rms^2 term) equals the derivative only for eps inside.
    rng = np.random.default_rng(3)
    n, eps = 6, 0.3
    x, dy, gamma = rng.standard_normal(n), rng.standard_normal(n), rng.uniform(0.5, 1.5, n)
    num = verify.numerical_grad(verify.vjp_loss(lambda z: specs.rmsnorm_forward(z, gamma, eps), dy), x, eps=1e-6)
    assert np.max(np.abs(specs.rmsnorm_backward(x, gamma, dy, eps) - num)) < 1e-8
    outside = lambda z: gamma * z / (math.sqrt(float(np.mean(z * z))) + eps)
    num_out = verify.numerical_grad(verify.vjp_loss(outside, dy), x, eps=1e-6)
    assert np.max(np.abs(specs.rmsnorm_backward(x, gamma, dy, eps) - num_out)) > 1e-3


def test_rmsnorm_single_element_closed_form():
    # n = 1: y = gamma*x/sqrt(x^2+eps) so dy/dx = gamma*eps/(x^2+eps)^(3/2).
    x, g, dy, eps = 1.7, 0.8, -1.3, 0.05
    dx = specs.rmsnorm_backward([x], [g], [dy], eps)[0]
    assert dx == pytest.approx(dy * g * eps / (x * x + eps) ** 1.5, rel=1e-13)


def test_rmsnorm_projection_identity():
    # x . dx = eps * c / r^3 with c = sum dy*gamma*x (follows from the formula's algebra).
    rng = np.random.default_rng(4)
    n, eps = 64, 1e-6
    x, dy, gamma = rng.standard_normal(n), rng.standard_normal(n), rng.uniform(0.5, 1.5, n)
    dx = specs.rmsnorm_backward(x, gamma, dy, eps)
    r = specs.rms(x, eps)
    c = np.sum(dy * gamma * x)
    assert np.dot(x, dx) == pytest.approx(eps * c / r ** 3, rel=1e-6, abs=1e-12)


def test_rmsnorm_rows_match_autograd():
    rng = np.random.default_rng(9)
    R, n, eps = 5, 40, 1e-6
    x, dy, gamma = rng.standard_normal((R, n)), rng.standard_normal((R, n)), rng.uniform(0.5, 1.5, n)
    xt = torch.tensor(x, requires_grad=True)
    y = torch.tensor(gamma) * xt / torch.sqrt((xt * xt).mean(-1, keepdim=True) + eps)
    (y * torch.tensor(dy)).sum().backward()
    np.testing.assert_allclose(rmsnorm_backward_rows(x, gamma, dy, eps), xt.grad.numpy(), rtol=0, atol=1e-12)


def test_scaled_dot_vjps_match_central_differences_and_fail_when_transposed():
    # scaledDotForward / scaledDotBackwardQ / scaledDotBackwardK ("Hesper.Training.VerifiedBackward",
    # section "Scaled Dot-Product"): the loss dscore * score differentiated by differences,
    # and the q and k gradients swapped (a plausible mistake) must not pass
    from oracle import verify
    rng = np.random.default_rng(31)
    q, k = rng.standard_normal(16), rng.standard_normal(16)
    sc, dscore = 0.25, -1.7
    num_q = verify.numerical_grad(lambda z: dscore * specs.scaled_dot_forward(z, k, sc), q, eps=1e-6)
    num_k = verify.numerical_grad(lambda z: dscore * specs.scaled_dot_forward(q, z, sc), k, eps=1e-6)
    np.testing.assert_allclose(specs.scaled_dot_backward_q(k, sc, dscore), num_q, rtol=1e-8, atol=1e-9)
    np.testing.assert_allclose(specs.scaled_dot_backward_k(q, sc, dscore), num_k, rtol=1e-8, atol=1e-9)
    assert np.max(np.abs(specs.scaled_dot_backward_q(q, sc, dscore) - num_q)) > 1e-2
    assert specs.scaled_dot_forward(q, k, sc) == pytest.approx(sc * float(np.sum(q * k)), rel=1e-14)
