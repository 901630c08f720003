"""Negative controls: the checker must reject the wrong backwards the Hesper commit log
lists (zero, identity, negated, wrong RoPE sign) and accept the correct ones."""

import numpy as np
import pytest

from oracle import attention as A
from oracle import specs, verify
from oracle.layer import rope_backward_rows, rope_forward_rows


WRONG = verify.wrong_backwards()


@pytest.mark.parametrize("kind", sorted(WRONG))
def test_softmax_wrong_backward_fails(kind):
    rng = np.random.default_rng(0)
    x, dy = rng.standard_normal(6), rng.standard_normal(6)
    num = verify.numerical_grad(verify.vjp_loss(specs.softmax_forward, dy), x)
    good = specs.softmax_backward(x, dy)
    assert verify.check_gradient(good, num)
    assert not verify.check_gradient(WRONG[kind](good, dy), num)


@pytest.mark.parametrize("kind", sorted(WRONG))
def test_rmsnorm_wrong_backward_fails(kind):
    rng = np.random.default_rng(1)
    x, dy, g = rng.standard_normal(8), rng.standard_normal(8), rng.uniform(0.5, 1.5, 8)
    num = verify.numerical_grad(verify.vjp_loss(lambda z: specs.rmsnorm_forward(z, g), dy), x)
    good = specs.rmsnorm_backward(x, g, dy)
    assert verify.check_gradient(good, num)
    assert not verify.check_gradient(WRONG[kind](good, dy), num)


@pytest.mark.parametrize("kind", sorted(WRONG) + ["wrong_rope_sign"])
def test_rope_wrong_backward_fails(kind):
    rng = np.random.default_rng(2)
    T, H, d = 2, 1, 64
    x, dy = rng.standard_normal((T, H, d)), rng.standard_normal((T, H, d))
    pos = np.array([5, 6])                      # pos 5: theta_0 = 5 rad, sin != 0
    num = verify.numerical_grad(verify.vjp_loss(lambda z: rope_forward_rows(z, pos), dy), x)
    good = rope_backward_rows(dy, pos)
    assert verify.check_gradient(good, num)
    bad = verify.rope_backward_wrong_sign(dy, pos) if kind == "wrong_rope_sign" else WRONG[kind](good, dy)
    assert not verify.check_gradient(bad, num)


@pytest.mark.parametrize("kind", sorted(WRONG))
def test_attention_wrong_backward_fails(kind):
    rng = np.random.default_rng(3)
    q, k, v, do = (rng.standard_normal(s) for s in [(1, 3, 1, 4), (1, 3, 1, 4), (1, 3, 1, 4), (1, 3, 1, 4)])
    sc = 0.5
    dq, _, _ = A.attention_backward(q, k, v, do, sc, True)
    num = verify.numerical_grad(lambda z: float(np.sum(do * A.attention_forward(z, k, v, sc, True)[0])), q)
    assert verify.check_gradient(dq, num)
    assert not verify.check_gradient(WRONG[kind](dq, do), num)


def test_checker_catches_planted_mistakes_in_attention():
    # Plausible slips in the chain (dropped D term, missing scale, transposed dS) must fail.
    rng = np.random.default_rng(4)
    q, k, v, do = (rng.standard_normal((1, 4, 1, 4)) for _ in range(4))
    sc = 0.6
    num = verify.numerical_grad(lambda z: float(np.sum(do * A.attention_forward(z, k, v, sc, True)[0])), q)
    S = sc * q[0, :, 0] @ k[0, :, 0].T
    S = np.where(np.tril(np.ones((4, 4), bool)), S, -np.inf)
    P = np.exp(S - S.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    dP = do[0, :, 0] @ v[0, :, 0].T
    D = np.sum(P * dP, 1, keepdims=True)
    good = sc * (P * (dP - D)) @ k[0, :, 0]
    assert verify.check_gradient(good.reshape(q.shape), num)
    for bad in (sc * (P * dP) @ k[0, :, 0],              # dropped D
                (P * (dP - D)) @ k[0, :, 0],             # missing scale
                sc * (P * (dP - D)).T @ k[0, :, 0]):     # transposed dS
        assert not verify.check_gradient(bad.reshape(q.shape), num)
