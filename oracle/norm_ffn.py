"""LayerNorm (no affine) and the FFN's ReLU^2 x Mul gate, forward and backward, in float64.
Test infrastructure only.

LayerNorm follows the DaisyChain-Train transformer.js page, functions ``lnFwd`` and
``lnBwd`` ("layernorm (no affine)"), per row of width C:
    mu = mean(x),  sigma = sqrt(mean((x - mu)^2) + 1e-5),  y = (x - mu) / sigma
    dx = (dy - mean(dy) - y * mean(dy * y)) / sigma
The backward takes the forward's y and sigma, as the page's does.

ReLU^2 x Mul follows the Hesper pull request's commit log ("FFN backward",
FFNBackward.lean): h = ReLU(gate)^2 * up elementwise, and
    dGate = dH * up * 2 * ReLU(gate),    dUp = dH * ReLU(gate)^2
"""

from __future__ import annotations

import numpy as np

LN_EPS = 1e-5   # the page's lnFwd adds 1e-5 inside the square root


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def layernorm_forward(x, eps: float = LN_EPS):
    """Rows of x [rows, C] -> (y [rows, C], sigma [rows])."""
    x = _f64(x)
    mu = x.mean(axis=1, keepdims=True)
    sig = np.sqrt(((x - mu) ** 2).mean(axis=1, keepdims=True) + eps)
    return (x - mu) / sig, sig[:, 0]


def layernorm_backward(dy, y, sig):
    """dx [rows, C] from the upstream gradient dy and the forward's y and sigma."""
    dy, y, sig = _f64(dy), _f64(y), _f64(sig)
    mdy = dy.mean(axis=1, keepdims=True)
    mdyy = (dy * y).mean(axis=1, keepdims=True)
    return (dy - mdy - y * mdyy) / sig[:, None]


def relu2_mul_forward(gate, up):
    """h = ReLU(gate)^2 * up, elementwise."""
    r = np.maximum(_f64(gate), 0.0)
    return r * r * _f64(up)


def relu2_mul_backward(gate, up, dh):
    """(dGate, dUp) of h = ReLU(gate)^2 * up for the upstream gradient dh."""
    r = np.maximum(_f64(gate), 0.0)
    dh, up = _f64(dh), _f64(up)
    return dh * up * 2.0 * r, dh * r * r
