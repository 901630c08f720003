"""Pins for the oracle's transformer attention block (LayerNorm, fused QKV projection,
causal multi-head attention with the saved softmax, output projection, residual):
central differences, torch float64 autograd of an independent forward, a single-token
closed form and planted mistakes."""

import numpy as np
import pytest
import torch

from oracle import block as BK
from oracle import verify


def _tiny(seed, B=2, T=3, H=2, d=4):
    rng = np.random.default_rng(seed)
    C = H * d
    return dict(xin=rng.standard_normal((B * T, C)) * 1.5 + 0.3, w_qkv=rng.standard_normal((C, 3 * C)) * 0.4,
                w_o=rng.standard_normal((C, C)) * 0.4), B, H, 1.0 / np.sqrt(d)


def _out(p, B, H, sc, causal=True, **over):
    q = dict(p, **over)
    return BK.block_forward(q["xin"], q["w_qkv"], q["w_o"], B, H, sc, causal)[0]


@pytest.mark.parametrize("causal", [True, False])
def test_block_backward_matches_central_differences(causal):
    p, B, H, sc = _tiny(31)
    dx2 = np.random.default_rng(32).standard_normal(p["xin"].shape)
    _, sv = BK.block_forward(p["xin"], p["w_qkv"], p["w_o"], B, H, sc, causal)
    got = BK.block_backward(sv, dx2, B, H, sc, causal)
    for name, g in zip(("xin", "w_qkv", "w_o"), got):
        num = verify.numerical_grad(lambda z: float(np.sum(dx2 * _out(p, B, H, sc, causal, **{name: z}))), p[name],
                                    eps=1e-6)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7, err_msg=name)


def test_block_backward_matches_torch_autograd():
    p, B, H, sc = _tiny(33, B=2, T=5, H=3, d=4)
    BT, C = p["xin"].shape
    T, d = BT // B, C // H
    dx2 = np.random.default_rng(34).standard_normal((BT, C))
    _, sv = BK.block_forward(p["xin"], p["w_qkv"], p["w_o"], B, H, sc)
    dx, gqkv, gwo = BK.block_backward(sv, dx2, B, H, sc)
    t = {k: torch.tensor(v, requires_grad=True) for k, v in p.items()}
    x = t["xin"]
    mu = x.mean(1, keepdim=True)
    y = (x - mu) / torch.sqrt(((x - mu) ** 2).mean(1, keepdim=True) + 1e-5)
    qkv = y @ t["w_qkv"]
    split = lambda z: z.reshape(B, T, H, d).permute(0, 2, 1, 3)           # [B, H, T, d]
    q, k, v = split(qkv[:, :C]), split(qkv[:, C:2 * C]), split(qkv[:, 2 * C:])
    s = (q @ k.transpose(-1, -2)) * sc
    s = s.masked_fill(~torch.tril(torch.ones(T, T, dtype=torch.bool)), float("-inf"))
    ctx = (torch.softmax(s, -1) @ v).permute(0, 2, 1, 3).reshape(BT, C)
    ((x + ctx @ t["w_o"]) * torch.tensor(dx2)).sum().backward()
    np.testing.assert_allclose(dx, t["xin"].grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(gqkv, t["w_qkv"].grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(gwo, t["w_o"].grad.numpy(), rtol=1e-11, atol=1e-12)


def test_block_single_token_closed_form():
    # T = 1: the softmax is the constant 1, so dS = 0 exactly: the q and k thirds of gWqkv
    # vanish, dv = dctx, and dln = dctx . Wv^T
    p, B, H, sc = _tiny(35, B=3, T=1, H=2, d=4)
    C = p["w_o"].shape[0]
    dx2 = np.random.default_rng(36).standard_normal(p["xin"].shape)
    _, sv = BK.block_forward(p["xin"], p["w_qkv"], p["w_o"], B, H, sc)
    dx, gqkv, gwo = BK.block_backward(sv, dx2, B, H, sc)
    np.testing.assert_array_equal(gqkv[:, :2 * C], 0.0)
    dctx = dx2 @ p["w_o"].T
    np.testing.assert_allclose(gqkv[:, 2 * C:], sv["ln_y"].T @ dctx, rtol=1e-13, atol=1e-14)
    from oracle.norm_ffn import layernorm_backward
    np.testing.assert_allclose(dx, dx2 + layernorm_backward(dctx @ p["w_qkv"][:, 2 * C:].T, sv["ln_y"], sv["ln_sig"]),
                               rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(gwo, sv["ctx"].T @ dx2, rtol=1e-13, atol=1e-14)


def test_block_planted_mistakes_fail_the_difference_check(monkeypatch):
    p, B, H, sc = _tiny(37)
    dx2 = np.random.default_rng(38).standard_normal(p["xin"].shape)
    _, sv = BK.block_forward(p["xin"], p["w_qkv"], p["w_o"], B, H, sc)
    num = verify.numerical_grad(lambda z: float(np.sum(dx2 * _out(p, B, H, sc, xin=z))), p["xin"], eps=1e-6)
    assert np.max(np.abs(BK.block_backward(sv, dx2, B, H, sc)[0] - num)) < 1e-6
    # the residual dropped
    assert np.max(np.abs(BK.block_backward(sv, dx2, B, H, sc)[0] - dx2 - num)) > 1e-3
    # dk and dv exchanged on their way into the QKV product
    real = BK.attention_backward
    monkeypatch.setattr(BK, "attention_backward", lambda *a, **k: (lambda r: (r[0], r[2], r[1]))(real(*a, **k)))
    assert np.max(np.abs(BK.block_backward(sv, dx2, B, H, sc)[0] - num)) > 1e-3
    monkeypatch.setattr(BK, "attention_backward", real)
    # LayerNorm backward skipped
    monkeypatch.setattr(BK, "layernorm_backward", lambda dy, y, s: np.asarray(dy))
    assert np.max(np.abs(BK.block_backward(sv, dx2, B, H, sc)[0] - num)) > 1e-3
