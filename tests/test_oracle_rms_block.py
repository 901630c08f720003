"""Pins for the oracle's Hesper-form attention layer (RMSNorm with gain, Q/K/V projections,
RoPE on queries and keys, causal attention with the saved softmax, output projection,
residual) and for its RMSNorm gain gradient: central differences, torch float64 autograd
of an independently written forward, a single-token closed form and planted mistakes."""

import numpy as np
import pytest
import torch

from oracle import rms_block as RB
from oracle import specs, verify


def _tiny(seed, B=2, T=3, H=2, d=4):
    rng = np.random.default_rng(seed)
    C = H * d
    return dict(x=rng.standard_normal((B * T, C)) * 1.5 + 0.3, gamma=rng.uniform(0.5, 1.5, C),
                w_qkv=rng.standard_normal((C, 3 * C)) * 0.4, w_o=rng.standard_normal((C, C)) * 0.4), B, H, 1.0 / np.sqrt(d)


def _out(p, B, H, sc, causal=True, layout=0, **over):
    q = dict(p, **over)
    return RB.rms_block_forward(q["x"], q["gamma"], q["w_qkv"], q["w_o"], B, H, sc, causal, layout=layout)[0]


def test_gamma_grad_matches_central_differences():
    # one RMSNorm over rows, scalar loss sum(dy o y): the gain gradient by differences
    rng = np.random.default_rng(40)
    x, g, dy = rng.standard_normal((5, 7)), rng.uniform(0.5, 1.5, 7), rng.standard_normal((5, 7))
    f = lambda gg: float(np.sum(dy * np.stack([specs.rmsnorm_forward(r, gg, 1e-6) for r in x])))
    np.testing.assert_allclose(RB.rmsnorm_gamma_grad(x, dy), verify.numerical_grad(f, g, eps=1e-6), rtol=1e-8,
                               atol=1e-9)


def test_gamma_grad_single_row_closed_form():
    # one row of constant magnitude: x = c * s with s_i = +-1 gives r = sqrt(c^2 + eps), so
    # dgamma_i = dy_i c s_i / sqrt(c^2 + eps)
    s = np.array([1.0, -1.0, 1.0, 1.0, -1.0, -1.0])
    c, eps = 0.75, 1e-6
    dy = np.arange(1.0, 7.0)
    got = RB.rmsnorm_gamma_grad((c * s)[None], dy[None], eps)
    np.testing.assert_allclose(got, dy * c * s / np.sqrt(c * c + eps), rtol=1e-14)


@pytest.mark.parametrize("causal,layout", [(True, 0), (False, 1)])
def test_rms_block_backward_matches_central_differences(causal, layout):
    p, B, H, sc = _tiny(41)
    dx2 = np.random.default_rng(42).standard_normal(p["x"].shape)
    _, sv = RB.rms_block_forward(p["x"], p["gamma"], p["w_qkv"], p["w_o"], B, H, sc, causal, layout=layout)
    got = RB.rms_block_backward(sv, dx2, B, H, sc, causal, layout=layout)
    for name, g in zip(("x", "gamma", "w_qkv", "w_o"), got):
        num = verify.numerical_grad(lambda z: float(np.sum(dx2 * _out(p, B, H, sc, causal, layout, **{name: z}))),
                                    p[name], eps=1e-6)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7, err_msg=name)


def _torch_rope(z, T, H, d, base=10000.0):
    # adjacent pairs (2i, 2i+1) rotated by theta = t base^(-2i/d), t the position in the sequence
    zz = z.reshape(-1, T, H, d // 2, 2)
    t = torch.arange(T, dtype=torch.float64)[:, None]
    th = t * base ** (-2.0 * torch.arange(d // 2, dtype=torch.float64)[None, :] / d)   # [T, d/2]
    c, s = torch.cos(th)[None, :, None, :], torch.sin(th)[None, :, None, :]
    z0, z1 = zz[..., 0], zz[..., 1]
    return torch.stack([z0 * c - z1 * s, z0 * s + z1 * c], dim=-1).reshape(z.shape)


def test_rms_block_backward_matches_torch_autograd():
    p, B, H, sc = _tiny(43, B=2, T=5, H=3, d=4)
    BT, C = p["x"].shape
    T, d = BT // B, C // H
    dx2 = np.random.default_rng(44).standard_normal((BT, C))
    _, sv = RB.rms_block_forward(p["x"], p["gamma"], p["w_qkv"], p["w_o"], B, H, sc)
    dx, dg, gqkv, gwo = RB.rms_block_backward(sv, dx2, B, H, sc)
    t = {k: torch.tensor(v, requires_grad=True) for k, v in p.items()}
    x = t["x"]
    n = t["gamma"] * x / torch.sqrt((x * x).mean(1, keepdim=True) + 1e-6)
    abv = n @ t["w_qkv"]
    q = _torch_rope(abv[:, :C], T, H, d).reshape(B, T, H, d).permute(0, 2, 1, 3)
    k = _torch_rope(abv[:, C:2 * C], T, H, d).reshape(B, T, H, d).permute(0, 2, 1, 3)
    v = abv[:, 2 * C:].reshape(B, T, H, d).permute(0, 2, 1, 3)
    s = (q @ k.transpose(-1, -2)) * sc
    s = s.masked_fill(~torch.tril(torch.ones(T, T, dtype=torch.bool)), float("-inf"))
    ctx = (torch.softmax(s, -1) @ v).permute(0, 2, 1, 3).reshape(BT, C)
    ((x + ctx @ t["w_o"]) * torch.tensor(dx2)).sum().backward()
    for name, g in (("x", dx), ("gamma", dg), ("w_qkv", gqkv), ("w_o", gwo)):
        np.testing.assert_allclose(g, t[name].grad.numpy(), rtol=1e-10, atol=1e-11, err_msg=name)


def test_rms_block_single_token_closed_form():
    # T = 1: the softmax is the constant 1 and the rotation angle is 0, so dS = 0: the q and
    # k thirds of gWqkv vanish, dn = dctx . Wv^T and dgamma = sum_t dn_t o x_t / r_t
    p, B, H, sc = _tiny(45, B=3, T=1, H=2, d=4)
    C = p["w_o"].shape[0]
    dx2 = np.random.default_rng(46).standard_normal(p["x"].shape)
    _, sv = RB.rms_block_forward(p["x"], p["gamma"], p["w_qkv"], p["w_o"], B, H, sc)
    dx, dg, gqkv, gwo = RB.rms_block_backward(sv, dx2, B, H, sc)
    np.testing.assert_array_equal(gqkv[:, :2 * C], 0.0)
    dn = (dx2 @ p["w_o"].T) @ p["w_qkv"][:, 2 * C:].T
    r = np.sqrt(np.mean(p["x"] ** 2, axis=1) + 1e-6)
    np.testing.assert_allclose(dg, np.sum(dn * p["x"] / r[:, None], axis=0), rtol=1e-12, atol=1e-13)
    n = p["gamma"] * p["x"] / r[:, None]
    np.testing.assert_allclose(gqkv[:, 2 * C:], n.T @ (dx2 @ p["w_o"].T), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gwo, sv["ctx"].T @ dx2, rtol=1e-13, atol=1e-14)


def test_rms_block_planted_mistakes_fail_the_difference_check(monkeypatch):
    p, B, H, sc = _tiny(47, T=4)
    dx2 = np.random.default_rng(48).standard_normal(p["x"].shape)
    _, sv = RB.rms_block_forward(p["x"], p["gamma"], p["w_qkv"], p["w_o"], B, H, sc)
    num_x = verify.numerical_grad(lambda z: float(np.sum(dx2 * _out(p, B, H, sc, x=z))), p["x"], eps=1e-6)
    num_g = verify.numerical_grad(lambda z: float(np.sum(dx2 * _out(p, B, H, sc, gamma=z))), p["gamma"], eps=1e-6)
    ok = RB.rms_block_backward(sv, dx2, B, H, sc)
    assert np.max(np.abs(ok[0] - num_x)) < 1e-6 and np.max(np.abs(ok[1] - num_g)) < 1e-6
    # dK passed to the projection without the inverse rotation
    real = RB._rope_seq
    calls = []

    def skip_second_backward(z, B_, T_, H_, d_, base, layout, backward):
        calls.append(backward)
        if backward and calls.count(True) == 2:
            return np.asarray(z, dtype=np.float64)
        return real(z, B_, T_, H_, d_, base, layout, backward)

    monkeypatch.setattr(RB, "_rope_seq", skip_second_backward)
    assert np.max(np.abs(RB.rms_block_backward(sv, dx2, B, H, sc)[0] - num_x)) > 1e-3
    monkeypatch.setattr(RB, "_rope_seq", real)
    # the forward rotation used for the backward of dq and dk (wrong sign of theta)
    monkeypatch.setattr(RB, "rope_backward_rows", RB.rope_forward_rows)
    assert np.max(np.abs(RB.rms_block_backward(sv, dx2, B, H, sc)[0] - num_x)) > 1e-3
    monkeypatch.undo()
    # the gain gradient without the 1/r of each row
    monkeypatch.setattr(RB, "rmsnorm_gamma_grad", lambda x, dy, eps=1e-6: np.sum(np.asarray(dy) * np.asarray(x), axis=0))
    assert np.max(np.abs(RB.rms_block_backward(sv, dx2, B, H, sc)[1] - num_g)) > 1e-3
