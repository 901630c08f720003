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

The FFN block built from these, with its two RMSNorms and three projections, is stated at
``ffn_forward`` below.
"""

from __future__ import annotations

import numpy as np

from .layer import linear_backward, rmsnorm_backward_rows, rmsnorm_forward_rows

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


# ----------------------------------------------------------------------------- FFN layer
#
# The FFN block of the Hesper commit log ("FFN backward", FFNBackward.lean), read as:
#     xn  = RMSNorm(x; gamma1)              ffnNorm
#     gu  = xn . Wgu,  Wgu = [Wgate | Wup]  ffnGate / ffnUp, one [C, 2F] product
#     h   = ReLU(gate)^2 * up               gate = gu[:, :F], up = gu[:, F:]
#     hn  = RMSNorm(h; gamma2)              ffnSubNorm
#     out = x + hn . Wdown                  ffnDown, with the residual
# and its backward in the commit log's op order (down transpose, sub-norm, ReLU^2 x Mul,
# gate/up transposes, norm), the residual passing dout through:
#     dhn, dWdown = dout . Wdown^T, hn^T . dout
#     dh          = RMSNormBackward(h, gamma2, dhn)
#     dgate, dup  = ReLU^2 x Mul backward(gate, up, dh)
#     dxn, dWgu   = [dgate | dup] . Wgu^T, xn^T . [dgate | dup]
#     dx          = dout + RMSNormBackward(x, gamma1, dxn)

def ffn_forward(x, gamma1, w_gu, gamma2, w_down, eps: float = 1e-6):
    """FFN block forward (reading above); returns (out, saved) with saved holding x,
    gamma1, xn, w_gu, gu, gamma2, hn, w_down."""
    x, w_gu, w_down = _f64(x), _f64(w_gu), _f64(w_down)
    F = w_gu.shape[1] // 2
    xn = rmsnorm_forward_rows(x, gamma1, eps)
    gu = xn @ w_gu
    h = relu2_mul_forward(gu[:, :F], gu[:, F:])
    hn = rmsnorm_forward_rows(h, gamma2, eps)
    saved = dict(x=x, gamma1=_f64(gamma1), xn=xn, w_gu=w_gu, gu=gu, gamma2=_f64(gamma2), hn=hn, w_down=w_down)
    return x + hn @ w_down, saved


def ffn_backward(saved, dout, eps: float = 1e-6):
    """FFN block backward from its saved tensors: returns (dx, dW_gu, dW_down).
    h is formed again from the saved gate and up (it is ReLU(gate)^2 * up)."""
    dout = _f64(dout)
    gu = _f64(saved["gu"])
    F = gu.shape[1] // 2
    gate, up = gu[:, :F], gu[:, F:]
    dhn, dw_down = linear_backward(saved["hn"], saved["w_down"], dout)
    dh = rmsnorm_backward_rows(relu2_mul_forward(gate, up), saved["gamma2"], dhn, eps)
    dgate, dup = relu2_mul_backward(gate, up, dh)
    dxn, dw_gu = linear_backward(saved["xn"], saved["w_gu"], np.concatenate([dgate, dup], axis=1))
    return dout + rmsnorm_backward_rows(saved["x"], saved["gamma1"], dxn, eps), dw_gu, dw_down
