"""One transformer attention block, forward and backward, in float64, as the
DaisyChain-Train transformer.js page builds it (functions ``init``-time layer loop of the
forward and ``backward``). Test infrastructure only.

Forward of one block over B sequences of T tokens, hidden C = H * d:
    ln   = LayerNorm(xin)             no affine (lnFwd): y and sigma kept
    q, k, v = ln.y . Wq, ln.y . Wk, ln.y . Wv      one [C, 3C] product with Wqkv = [Wq | Wk | Wv]
    P    = causal softmax(scale q_h . k_h^T) per (sequence, head), kept (aAll)
    ctx  = P . v_h per head, scattered back to [B T, C]
    x2   = xin + ctx . Wo
Backward from dx2 (the page's order):
    gWo, dctx   = ctx^T . dx2, dx2 . Wo^T
    dv, dq, dk  = P^T . dctx_h,  scale dS . k_h,  scale dS^T . q_h   with dS = P o (dP - rowsum(P o dP)),
                  dP = dctx_h . v_h^T, per head (the attention backward of the same page)
    gWqkv       = ln.y^T . [dq | dk | dv]
    dln         = dq . Wq^T + dk . Wk^T + dv . Wv^T = [dq | dk | dv] . Wqkv^T
    dx          = dx2 + lnBwd(dln, ln.y, sigma)
"""

from __future__ import annotations

import numpy as np

from .attention import attention_backward, attention_forward
from .layer import linear_backward
from .norm_ffn import layernorm_backward, layernorm_forward


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def block_forward(xin, w_qkv, w_o, B: int, H: int, scale: float, causal: bool = True):
    """xin [B*T, C], w_qkv [C, 3C], w_o [C, C] -> (x2, saved); saved holds ln_y, ln_sig,
    w_qkv, qkv [B*T, 3C], P [B*H, T, T], ctx [B*T, C], w_o."""
    xin, w_qkv, w_o = _f64(xin), _f64(w_qkv), _f64(w_o)
    BT, C = xin.shape
    T, d = BT // B, C // H
    y, sig = layernorm_forward(xin)
    qkv = y @ w_qkv
    heads = lambda z: z.reshape(B, T, H, d)
    ctx, _lse, P = attention_forward(heads(qkv[:, :C]), heads(qkv[:, C:2 * C]), heads(qkv[:, 2 * C:]), scale, causal,
                                     want_p=True)
    ctx = ctx.reshape(BT, C)
    saved = dict(ln_y=y, ln_sig=sig, w_qkv=w_qkv, qkv=qkv, P=P.reshape(B * H, T, T), ctx=ctx, w_o=w_o)
    return xin + ctx @ w_o, saved


def block_backward(saved, dx2, B: int, H: int, scale: float, causal: bool = True):
    """Backward of one block from its saved tensors: returns (dx, gW_qkv, gW_o)."""
    dx2 = _f64(dx2)
    BT, C = dx2.shape
    T, d = BT // B, C // H
    dctx, gwo = linear_backward(saved["ctx"], saved["w_o"], dx2)
    qkv = _f64(saved["qkv"])
    heads = lambda z: z.reshape(B, T, H, d)
    dq, dk, dv = attention_backward(heads(qkv[:, :C]), heads(qkv[:, C:2 * C]), heads(qkv[:, 2 * C:]), heads(dctx),
                                    scale, causal, P=_f64(saved["P"]).reshape(B, H, T, T))
    dqkv = np.concatenate([dq.reshape(BT, C), dk.reshape(BT, C), dv.reshape(BT, C)], axis=1)
    dln, gwqkv = linear_backward(saved["ln_y"], saved["w_qkv"], dqkv)
    return dx2 + layernorm_backward(dln, saved["ln_y"], saved["ln_sig"]), gwqkv, gwo
