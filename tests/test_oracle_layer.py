"""Pins for the oracle's linear backward, one-layer backward and the layer stack."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import layer as L
from oracle import verify


def test_linear_hand_fixture(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "linear_hand.json")))
    dx, dw = L.linear_backward(g["x"], g["w"], g["dy"])
    np.testing.assert_array_equal(dx, g["dx"])
    np.testing.assert_array_equal(dw, g["dw"])


def test_linear_outer_product_form_and_transpose_identity():
    # dW = sum_t x_t (x) dy_t; <dX, X> = <dW, W> = <dY, X.W> ("self-consistent with transpose").
    rng = np.random.default_rng(1)
    x, w, dy = rng.standard_normal((5, 7)), rng.standard_normal((7, 3)), rng.standard_normal((5, 3))
    dx, dw = L.linear_backward(x, w, dy)
    dx2, dw2 = L.linear_backward_outer(x, w, dy)
    np.testing.assert_allclose(dw, dw2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dx, dx2, rtol=0, atol=0)
    ref = np.sum(dy * (x @ w))
    assert np.sum(dx * x) == pytest.approx(ref, rel=1e-12)
    assert np.sum(dw * w) == pytest.approx(ref, rel=1e-12)


def test_linear_fd_and_autograd():
    rng = np.random.default_rng(2)
    x, w, dy = rng.standard_normal((4, 3)), rng.standard_normal((3, 5)), rng.standard_normal((4, 5))
    dx, dw = L.linear_backward(x, w, dy)
    assert verify.check_gradient(dx, verify.numerical_grad(verify.vjp_loss(lambda z: z @ w, dy), x))
    assert verify.check_gradient(dw, verify.numerical_grad(verify.vjp_loss(lambda z: x @ z, dy), w))
    xt, wt = torch.tensor(x, requires_grad=True), torch.tensor(w, requires_grad=True)
    ((xt @ wt) * torch.tensor(dy)).sum().backward()
    np.testing.assert_allclose(dx, xt.grad.numpy(), atol=1e-13)
    np.testing.assert_allclose(dw, wt.grad.numpy(), atol=1e-13)


def _tiny_layer(seed, T=4, H=2, d=8):
    rng = np.random.default_rng(seed)
    C = H * d
    return dict(h=rng.standard_normal((T, C)), gamma=rng.uniform(0.5, 1.5, C),
                K=rng.standard_normal((T, H, d)), V=rng.standard_normal((T, H, d)),
                W=rng.standard_normal((C, C)) * 0.3), H, 1.0 / np.sqrt(d)


def test_layer_backward_fd():
    p, H, sc = _tiny_layer(3)
    T, C = p["h"].shape
    g = np.random.default_rng(4).standard_normal((T, C))
    _, saved = L.layer_forward(p["h"], p["gamma"], p["K"], p["V"], p["W"], H, sc)
    g_in, dW, dK, dV = L.layer_backward(saved, g, H, sc)

    def out_of(h=p["h"], K=p["K"], V=p["V"], W=p["W"]):
        return L.layer_forward(h, p["gamma"], K, V, W, H, sc)[0]

    assert verify.check_gradient(g_in, verify.numerical_grad(verify.vjp_loss(lambda z: out_of(h=z), g), p["h"]))
    assert verify.check_gradient(dW, verify.numerical_grad(verify.vjp_loss(lambda z: out_of(W=z), g), p["W"]))
    assert verify.check_gradient(dK, verify.numerical_grad(verify.vjp_loss(lambda z: out_of(K=z), g), p["K"]))
    assert verify.check_gradient(dV, verify.numerical_grad(verify.vjp_loss(lambda z: out_of(V=z), g), p["V"]))
    # tighter: central differences are O(eps^2) accurate
    num = verify.numerical_grad(verify.vjp_loss(lambda z: out_of(h=z), g), p["h"], eps=1e-5)
    assert np.max(np.abs(g_in - num)) < 1e-7


def test_layer_backward_matches_autograd():
    p, H, sc = _tiny_layer(5, T=6, H=2, d=8)
    T, C = p["h"].shape
    d = C // H
    g = np.random.default_rng(6).standard_normal((T, C))
    _, saved = L.layer_forward(p["h"], p["gamma"], p["K"], p["V"], p["W"], H, sc)
    g_in, dW, dK, dV = L.layer_backward(saved, g, H, sc)
    # independent torch forward: rmsnorm -> rope (complex rotation) -> causal attention -> h + o W
    ht = torch.tensor(p["h"], requires_grad=True)
    Wt = torch.tensor(p["W"], requires_grad=True)
    Kt = torch.tensor(p["K"], requires_grad=True)
    Vt = torch.tensor(p["V"], requires_grad=True)
    n = torch.tensor(p["gamma"]) * ht / torch.sqrt((ht * ht).mean(-1, keepdim=True) + 1e-6)
    n = n.reshape(T, H, d)
    inv = 10000.0 ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    th = torch.arange(T, dtype=torch.float64)[:, None, None] * inv[None, None, :]
    z = torch.complex(n[..., 0::2], n[..., 1::2]) * torch.polar(torch.ones_like(th), th)
    q = torch.stack([z.real, z.imag], -1).reshape(T, H, d)
    s = torch.einsum("ihd,jhd->hij", q, Kt) * sc
    s = s.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
    o = torch.einsum("hij,jhd->ihd", torch.softmax(s, -1), Vt).reshape(T, C)
    out = ht + o @ Wt
    (out * torch.tensor(g)).sum().backward()
    np.testing.assert_allclose(g_in, ht.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dK, Kt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dV, Vt.grad.numpy(), atol=1e-11)


def test_two_layer_stack_is_chain_rule_composition():
    p0, H, sc = _tiny_layer(7)
    p1, _, _ = _tiny_layer(8)
    T, C = p0["h"].shape
    dy = np.random.default_rng(9).standard_normal((T, C))

    def stack_fwd(h):
        o0, s0 = L.layer_forward(h, p0["gamma"], p0["K"], p0["V"], p0["W"], H, sc)
        o1, s1 = L.layer_forward(o0, p1["gamma"], p1["K"], p1["V"], p1["W"], H, sc)
        return o1, [s0, s1]

    _, saved = stack_fwd(p0["h"])
    g0, grads = L.stack_backward(saved, dy, H, sc)
    num = verify.numerical_grad(verify.vjp_loss(lambda z: stack_fwd(z)[0], dy), p0["h"], eps=1e-5)
    assert verify.check_gradient(g0, num)
    assert np.max(np.abs(g0 - num)) < 1e-7
