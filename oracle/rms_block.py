"""One attention layer of the Hesper form, forward and backward, in float64: RMSNorm with a
learned gain, Q/K/V projections, RoPE on the projected queries and keys, causal multi-head
attention, output projection and residual. Test infrastructure only.

The pieces are the pages' own: rmsNormForward / rmsNormBackward and ropeForward /
ropeBackward of "Hesper.Training.VerifiedBackward" (sections "RMSNorm" and "RoPE (Rotary
Position Embedding)"), the attention chain of its section "Attention (full single-head)"
batched with the causal mask of the DaisyChain-Train transformer.js `backward`, and the
fused Q/K/V weight gradient of that same `backward` (one left operand ln^T for the three
weight gradients, the three input-gradient terms summed). How they are put together is a
reading: no page prints this layer whole. Per sequence of T tokens (B sequences), hidden
C = H d, positions t = 0 .. T-1 within each sequence:
    r_t = sqrt(mean(x_t^2) + eps),  n_t = gamma o x_t / r_t         (rmsNormForward per row)
    [a | b | v] = n . Wqkv                                           (Wqkv = [Wq | Wk | Wv], [C, 3C])
    q = RoPE(a), k = RoPE(b)     per head, adjacent pairs (2i, 2i+1) or split halves
    P = causal softmax(scale q_h . k_h^T),  ctx = P v_h,  x2 = x + ctx . Wo
Backward from dx2:
    gWo, dctx  = ctx^T dx2, dx2 Wo^T
    dq, dk, dv = attention backward with the saved P
    da, db     = RoPEBackward(dq), RoPEBackward(dk)                  (rotation by -theta)
    gWqkv, dn  = n^T [da | db | dv], [da | db | dv] Wqkv^T
    dx         = dx2 + RMSNormBackward(x, gamma, dn)
    dgamma     = sum_t dn_t o x_t / r_t
The page's rmsNormBackward returns dx only; dgamma is the same map's derivative in gamma:
n_t depends on gamma_i only through gamma_i x_ti / r_t, so dL/dgamma_i = sum_t dn_ti x_ti / r_t.
"""

from __future__ import annotations

import numpy as np

from . import specs
from .attention import attention_backward, attention_forward
from .layer import linear_backward, rmsnorm_backward_rows, rmsnorm_forward_rows, rope_backward_rows, rope_forward_rows


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def rmsnorm_gamma_grad(x, dy, eps: float = 1e-6) -> np.ndarray:
    """dgamma of rmsNormForward applied to every row of x [rows, n], upstream dy [rows, n]:
    sum over rows of dy o x / r (r per row, as in specs.rms)."""
    x, dy = _f64(x), _f64(dy)
    r = np.array([specs.rms(row, eps) for row in x])
    return np.sum(dy * x / r[:, None], axis=0)


def _rope_seq(z, B: int, T: int, H: int, d: int, base: float, layout: int, backward: bool) -> np.ndarray:
    """RoPE (or its backward) on z [B T, H d] viewed per sequence as [T, H, d], positions 0 .. T-1."""
    z = _f64(z).reshape(B, T, H, d)
    f = rope_backward_rows if backward else rope_forward_rows
    return np.stack([f(z[b], np.arange(T), base, layout) for b in range(B)]).reshape(B * T, H * d)


def rms_block_forward(x, gamma, w_qkv, w_o, B: int, H: int, scale: float, causal: bool = True, eps: float = 1e-6,
                      base: float = 10000.0, layout: int = 0):
    """x [B T, C], gamma [C], w_qkv [C, 3C], w_o [C, C] -> (x2, saved); saved holds x, gamma,
    n [B T, C], w_qkv, qkv [B T, 3C] (rotated q and k, then v), P [B H, T, T], ctx [B T, C], w_o."""
    x, gamma, w_qkv, w_o = _f64(x), _f64(gamma), _f64(w_qkv), _f64(w_o)
    BT, C = x.shape
    T, d = BT // B, C // H
    n = rmsnorm_forward_rows(x, gamma, eps)
    abv = n @ w_qkv
    q = _rope_seq(abv[:, :C], B, T, H, d, base, layout, backward=False)
    k = _rope_seq(abv[:, C:2 * C], B, T, H, d, base, layout, backward=False)
    v = abv[:, 2 * C:]
    heads = lambda z: z.reshape(B, T, H, d)
    ctx, _lse, P = attention_forward(heads(q), heads(k), heads(v), scale, causal, want_p=True)
    ctx = ctx.reshape(BT, C)
    saved = dict(x=x, gamma=gamma, n=n, w_qkv=w_qkv, qkv=np.concatenate([q, k, v], axis=1),
                 P=P.reshape(B * H, T, T), ctx=ctx, w_o=w_o)
    return x + ctx @ w_o, saved


def rms_block_backward(saved, dx2, B: int, H: int, scale: float, causal: bool = True, eps: float = 1e-6,
                       base: float = 10000.0, layout: int = 0):
    """Backward of one layer from its saved tensors: returns (dx, dgamma, gW_qkv, gW_o)."""
    dx2 = _f64(dx2)
    BT, C = dx2.shape
    T, d = BT // B, C // H
    dctx, gwo = linear_backward(saved["ctx"], saved["w_o"], dx2)
    qkv = _f64(saved["qkv"])
    heads = lambda z: z.reshape(B, T, H, d)
    dq, dk, dv = attention_backward(heads(qkv[:, :C]), heads(qkv[:, C:2 * C]), heads(qkv[:, 2 * C:]), heads(dctx),
                                    scale, causal, P=_f64(saved["P"]).reshape(B, H, T, T))
    da = _rope_seq(dq.reshape(BT, C), B, T, H, d, base, layout, backward=True)
    db = _rope_seq(dk.reshape(BT, C), B, T, H, d, base, layout, backward=True)
    dabv = np.concatenate([da, db, dv.reshape(BT, C)], axis=1)
    dn, gwqkv = linear_backward(saved["n"], saved["w_qkv"], dabv)
    dx = dx2 + rmsnorm_backward_rows(saved["x"], saved["gamma"], dn, eps)
    return dx, rmsnorm_gamma_grad(saved["x"], dn, eps), gwqkv, gwo
