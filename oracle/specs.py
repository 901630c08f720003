"""Single-vector forward/backward specs, as stated on the "Hesper.Training.VerifiedBackward"
API page. Test infrastructure only (see the package docstring).

Each function is written from the page's formula; where the page leaves the body
unrendered (softmaxForward, rmsNormForward, attentionForward, the numerical checks) the
plainest reading is taken and stated in the docstring.
"""

from __future__ import annotations

import math

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------- softmax

def softmax_forward(x) -> np.ndarray:
    """Section "Softmax", softmaxForward (body unrendered on the page).

    Reading: s_i = exp(x_i) / sum_j exp(x_j); the maximum is subtracted first, which
    changes nothing mathematically and keeps exp finite.
    """
    x = _f64(x)
    e = np.exp(x - np.max(x))
    return e / np.sum(e)


def softmax_backward(x, dy) -> np.ndarray:
    """Section "Softmax", softmaxBackward: dx_i = s_i * (dy_i - sum_j s_j * dy_j)."""
    s = softmax_forward(x)
    dy = _f64(dy)
    return s * (dy - np.sum(s * dy))


def softmax_backward_sums_to_zero(x, dy) -> float:
    """Section "Softmax", softmaxBackwardSumsToZero: the plain left-to-right sum of the
    backward result (zero up to rounding, because the outputs of softmax sum to one)."""
    total = 0.0
    for v in softmax_backward(x, dy):
        total += float(v)
    return total


# ----------------------------------------------------------------------------- RoPE

def rope_forward(x0, x1, theta):
    """Section "RoPE (Rotary Position Embedding)", ropeForward: rotate (x0, x1) by theta."""
    x0, x1, theta = _f64(x0), _f64(x1), _f64(theta)
    c, s = np.cos(theta), np.sin(theta)
    return x0 * c - x1 * s, x0 * s + x1 * c


def rope_backward(dy0, dy1, theta):
    """Section "RoPE (Rotary Position Embedding)", ropeBackward: the inverse rotation
    R(-theta): (dy0 cos + dy1 sin, -dy0 sin + dy1 cos)."""
    dy0, dy1, theta = _f64(dy0), _f64(dy1), _f64(theta)
    c, s = np.cos(theta), np.sin(theta)
    return dy0 * c + dy1 * s, -dy0 * s + dy1 * c


def rope_roundtrip_check(x0, x1, theta, tol: float = 1e-6) -> bool:
    """Section "RoPE", ropeRoundtripCheck: backward(forward(x)) returns x within tol.

    Reading of the unrendered body: both components agree within the absolute tol.
    """
    y0, y1 = rope_forward(x0, x1, theta)
    z0, z1 = rope_backward(y0, y1, theta)
    return bool(np.all(np.abs(z0 - _f64(x0)) <= tol) and np.all(np.abs(z1 - _f64(x1)) <= tol))


def rope_angles(pos, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """Rotation angle of pair i at position p: theta = p * base^(-2i/head_dim).

    The frequency law is the one the single-query workload states (theta_i =
    pos * 10000^(-2i/64) for 32 pairs); the pages do not print it for other head sizes,
    so the same law with head_dim in place of 64 is used. Returns [len(pos), head_dim/2].
    """
    pos = np.atleast_1d(_f64(pos))
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = np.power(float(base), -2.0 * i / head_dim)
    return pos[:, None] * inv_freq[None, :]


# ----------------------------------------------------------------------------- RMSNorm

def rms(x, eps: float = 1e-6) -> float:
    """r = sqrt(mean(x^2) + eps).

    Reading of the unrendered rmsNormForward: eps sits inside the square root. This is
    the reading under which the page's backward (with its n * rms^2 term) is the exact
    derivative; a tight finite-difference test pins it.
    """
    x = _f64(x)
    return math.sqrt(float(np.mean(x * x)) + eps)


def rmsnorm_forward(x, gamma, eps: float = 1e-6) -> np.ndarray:
    """Section "RMSNorm", rmsNormForward: y_i = gamma_i * x_i / rms(x)."""
    return _f64(gamma) * _f64(x) / rms(x, eps)


def rmsnorm_backward(x, gamma, dy, eps: float = 1e-6) -> np.ndarray:
    """Section "RMSNorm", rmsNormBackward:
    dx_i = (1/rms) * (dy_i * gamma_i - x_i * sum_j(dy_j * gamma_j * x_j) / (n * rms^2))."""
    x, gamma, dy = _f64(x), _f64(gamma), _f64(dy)
    n = x.shape[0]
    r = rms(x, eps)
    c = float(np.sum(dy * gamma * x))
    return (dy * gamma - x * c / (n * r * r)) / r


# ----------------------------------------------------------------------------- scaled dot

def dot_product(a, b) -> float:
    """Section "Scaled Dot-Product", dotProduct: left fold of elementwise products."""
    total = 0.0
    for x, y in zip(_f64(a), _f64(b)):
        total += float(x) * float(y)
    return total


def scaled_dot_forward(q, k, scale: float) -> float:
    """scaledDotForward: score = scale * q . k."""
    return scale * dot_product(q, k)


def scaled_dot_backward_q(k, scale: float, dscore: float) -> np.ndarray:
    """scaledDotBackwardQ: dq = scale * dScore * k."""
    return _f64(k) * scale * dscore


def scaled_dot_backward_k(q, scale: float, dscore: float) -> np.ndarray:
    """scaledDotBackwardK: dk = scale * dScore * q."""
    return _f64(q) * scale * dscore


# ----------------------------------------------------------------------------- single-head attention

def attention_scores(q, k_cache, scale: float) -> np.ndarray:
    return np.array([scaled_dot_forward(q, k_s, scale) for k_s in _f64(k_cache)])


def attention_forward(q, k_cache, v_cache, scale: float) -> np.ndarray:
    """Section "Attention (full single-head)", attentionForward:
    out[d] = sum_s softmax(scale * q . K[s])_s * V[s][d]."""
    attn = softmax_forward(attention_scores(q, k_cache, scale))
    v = _f64(v_cache)
    out = np.zeros(v.shape[1])
    for s in range(v.shape[0]):
        out += attn[s] * v[s]
    return out


def attention_backward_q(q, k_cache, v_cache, scale: float, dout) -> np.ndarray:
    """attentionBackwardQ, the page's three steps:
      1. dAttn[s] = sum_d dOut[d] * V[s][d]
      2. dScores = softmax_backward(scores, dAttn)
      3. dQ[d] = scale * sum_s dScores[s] * K[s][d]
    """
    k, v = _f64(k_cache), _f64(v_cache)
    scores = attention_scores(q, k, scale)
    d_attn = np.array([dot_product(dout, v[s]) for s in range(v.shape[0])])
    d_scores = softmax_backward(scores, d_attn)
    dq = np.zeros(k.shape[1])
    for s in range(k.shape[0]):
        dq += scaled_dot_backward_q(k[s], scale, d_scores[s])
    return dq


def attention_backward_k(q, k_cache, v_cache, scale: float, dout) -> np.ndarray:
    """dK[s] = scale * dScores[s] * q: scaledDotBackwardK applied at every cache row with
    the dScores of attentionBackwardQ (the page defines the atom; the composition is the
    chain rule through score_s = scale * q . K[s])."""
    k, v = _f64(k_cache), _f64(v_cache)
    scores = attention_scores(q, k, scale)
    d_attn = np.array([dot_product(dout, v[s]) for s in range(v.shape[0])])
    d_scores = softmax_backward(scores, d_attn)
    return np.stack([scaled_dot_backward_k(q, scale, d_scores[s]) for s in range(k.shape[0])])


def attention_backward_v(q, k_cache, scale: float, dout) -> np.ndarray:
    """attentionBackwardV: dV[s][d] = attn[s] * dOut[d] (needs no V)."""
    attn = softmax_forward(attention_scores(q, k_cache, scale))
    return np.outer(attn, _f64(dout))
