"""Linear backward, row-wise RoPE and RMSNorm backward, one attention layer's backward
and the reverse layer stack, in float64. Test infrastructure only.

Layer reading (the pages fix the backward chain, not a full layer definition):
    n   = RMSNorm(h; gamma, eps)                 per token row of width C = H * d
    q   = RoPE(n viewed as [T, H, d]; pos = t)   adjacent pairs (2i, 2i+1)
    o   = Attention(q, K, V; P saved)            K, V are the layer's saved caches
    out = h + o . W                              residual plus linear (Y = X . W)
Backward, as the Hesper commit log orders it (linear, attention, RoPE, RMSNorm; the
residual passes the hidden gradient through unchanged; the 30 layers run in reverse):
    dO, dW   = g . W^T, o^T . g
    dq, dK, dV = attention backward with the saved softmax P
    g_in     = g + RMSNormBackward(h, gamma, RoPEBackward(dq))
"""

from __future__ import annotations

import numpy as np

from . import specs
from .attention import attention_backward, attention_forward


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------- linear

def linear_forward(x, w) -> np.ndarray:
    """Y = X . W with X [T, K], W [K, N]."""
    return _f64(x) @ _f64(w)


def linear_backward(x, w, dy):
    """Linear backward of Y = X . W (Hesper commit log: "outer product dW + transpose dX";
    transformer.js backward: gWo = ctxOut^T . dx2, dctx = dx2 . Wo^T):
        dX = dY . W^T
        dW = X^T . dY = sum over tokens t of the outer product x_t (x) dy_t
    """
    x, w, dy = _f64(x), _f64(w), _f64(dy)
    return dy @ w.T, x.T @ dy


def linear_backward_outer(x, w, dy):
    """The same dW written as the literal sum of per-token outer products (for checks)."""
    x, dy = _f64(x), _f64(dy)
    dw = np.zeros((x.shape[1], dy.shape[1]))
    for t in range(x.shape[0]):
        dw += np.outer(x[t], dy[t])
    return _f64(dy) @ _f64(w).T, dw


# ----------------------------------------------------------------------------- row-wise RoPE

def _pair_index(head_dim: int, layout: int):
    half = head_dim // 2
    i = np.arange(half)
    if layout == 0:              # adjacent pairs (2i, 2i+1)
        return 2 * i, 2 * i + 1
    if layout == 1:              # split halves (i, i + d/2)
        return i, i + half
    raise ValueError("layout must be 0 (adjacent pairs) or 1 (split halves)")


def rope_forward_rows(x, pos, base: float = 10000.0, layout: int = 0) -> np.ndarray:
    """Apply ropeForward to every pair of x [T, H, d]; token t uses position pos[t]."""
    x = _f64(x)
    T, H, d = x.shape
    theta = specs.rope_angles(pos, d, base)[:, None, :]      # [T, 1, d/2]
    a, b = _pair_index(d, layout)
    y = np.empty_like(x)
    y[..., a], y[..., b] = specs.rope_forward(x[..., a], x[..., b], theta)
    return y


def rope_backward_rows(dy, pos, base: float = 10000.0, layout: int = 0) -> np.ndarray:
    """Apply ropeBackward (R(-theta)) to every pair of dy [T, H, d]."""
    dy = _f64(dy)
    T, H, d = dy.shape
    theta = specs.rope_angles(pos, d, base)[:, None, :]
    a, b = _pair_index(d, layout)
    dx = np.empty_like(dy)
    dx[..., a], dx[..., b] = specs.rope_backward(dy[..., a], dy[..., b], theta)
    return dx


# ----------------------------------------------------------------------------- row-wise RMSNorm

def rmsnorm_forward_rows(x, gamma, eps: float = 1e-6) -> np.ndarray:
    x = _f64(x)
    return np.stack([specs.rmsnorm_forward(row, gamma, eps) for row in x])


def rmsnorm_backward_rows(x, gamma, dy, eps: float = 1e-6) -> np.ndarray:
    x, dy = _f64(x), _f64(dy)
    return np.stack([specs.rmsnorm_backward(x[r], gamma, dy[r], eps) for r in range(x.shape[0])])


# ----------------------------------------------------------------------------- layer

def layer_saved(h, gamma, K, V, W, H: int, scale: float, eps: float = 1e-6,
                base: float = 10000.0, causal: bool = True, layout: int = 0):
    """The tensors one layer's backward reads, from its forward (module docstring):
    x (= h), gamma, W, o, q, K, V, P."""
    h = _f64(h)
    T, C = h.shape
    d = C // H
    n = rmsnorm_forward_rows(h, gamma, eps)
    q = rope_forward_rows(n.reshape(T, H, d), np.arange(T), base, layout)
    O, _lse, P = attention_forward(q[None], _f64(K)[None], _f64(V)[None], scale, causal, want_p=True)
    o = O[0].reshape(T, C)
    return dict(x=h, gamma=_f64(gamma), W=_f64(W), o=o, q=q, K=_f64(K), V=_f64(V), P=P[0])


def layer_forward(h, gamma, K, V, W, H: int, scale: float, eps: float = 1e-6,
                  base: float = 10000.0, causal: bool = True, layout: int = 0):
    """Forward of one layer (module docstring); returns (out, saved)."""
    saved = layer_saved(h, gamma, K, V, W, H, scale, eps, base, causal, layout)
    return saved["x"] + linear_forward(saved["o"], W), saved


def layer_backward(saved, g, H: int, scale: float, eps: float = 1e-6,
                   base: float = 10000.0, causal: bool = True, layout: int = 0, want_dw: bool = True):
    """Backward of one layer: returns (g_in, dW, dK, dV); dW is None when not wanted."""
    g = _f64(g)
    T, C = g.shape
    d = C // H
    if want_dw:
        d_o, dW = linear_backward(saved["o"], saved["W"], g)
    else:
        d_o, dW = g @ saved["W"].T, None
    dq, dK, dV = attention_backward(saved["q"][None], saved["K"][None], saved["V"][None],
                                    d_o.reshape(1, T, H, d), scale, causal, P=saved["P"][None])
    dn = rope_backward_rows(dq[0], np.arange(T), base, layout)
    dh = rmsnorm_backward_rows(saved["x"], saved["gamma"], dn.reshape(T, C), eps)
    return g + dh, dW, dK[0], dV[0]


def stack_backward(saved_layers, dy, H: int, scale: float, eps: float = 1e-6,
                   base: float = 10000.0, causal: bool = True, layout: int = 0):
    """Run layer_backward from the last layer to the first; returns (g_0, per-layer grads)."""
    g = _f64(dy)
    grads = [None] * len(saved_layers)
    for l in reversed(range(len(saved_layers))):
        g, dW, dK, dV = layer_backward(saved_layers[l], g, H, scale, eps, base, causal, layout)
        grads[l] = dict(dW=dW, dK=dK, dV=dV, g_in=g)
    return g, grads
