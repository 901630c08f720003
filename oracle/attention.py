"""Batched multi-head attention forward and backward in float64. Test infrastructure only.

Shapes follow the [B, T, H, d] activation layout: q, dout [B, Tq, Hq, d]; k, v
[B, Tk, Hkv, d]; lse [B, Hq, Tq]; P [B, Hq, Tq, Tk].

The backward is the chain the "Hesper.Training.VerifiedBackward" page states for one
query (section "Attention (full single-head)", attentionBackwardQ/V, built from
softmaxBackward and scaledDotBackwardQ/K), applied to every query row of every head:
    dP = dO . V^T            (dAttn[s] = sum_d dOut[d] V[s][d])
    D  = rowsum(P o dP)
    dS = P o (dP - D)        (softmaxBackward)
    dQ = scale * dS . K      (scaledDotBackwardQ summed over keys)
    dK = scale * dS^T . Q    (scaledDotBackwardK summed over queries and the group's heads)
    dV = P^T . dO            (attentionBackwardV summed over queries and the group's heads)
The batched causal form (key tj visible to query ti iff tj <= ti) is the one of the
DaisyChain-Train transformer.js page, function ``backward``; with Tq != Tk the mask is
aligned bottom-right: key j is visible to query i iff j <= i + (Tk - Tq).

Grouped queries: q-head h reads kv-head h // (Hq // Hkv); the pages do not state a
mapping, consecutive grouping is taken. Rows are processed in blocks only to bound
memory; no other reordering is done.
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def visible_keys(Tq: int, Tk: int, causal: bool, rows=None) -> np.ndarray:
    """Boolean [len(rows), Tk]: True where key j is visible to query i."""
    rows = np.arange(Tq) if rows is None else np.asarray(rows)
    j = np.arange(Tk)
    if not causal:
        return np.ones((rows.shape[0], Tk), dtype=bool)
    return j[None, :] <= rows[:, None] + (Tk - Tq)


def _group(Hq: int, Hkv: int) -> int:
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return Hq // Hkv


def _key_limit(i1: int, Tq: int, Tk: int, causal: bool) -> int:
    """Number of leading keys any row below i1 can see."""
    return Tk if not causal else max(0, min(Tk, i1 + Tk - Tq))


def attention_forward(q, k, v, scale: float, causal: bool, want_p: bool = False, row_block: int = 1024):
    """O = softmax(scale * Q K^T) V per head (section "Attention (full single-head)",
    attentionForward), with LSE_i = ln sum_{visible j} exp(scale * q_i . k_j).

    Returns (O [B,Tq,Hq,d], lse [B,Hq,Tq]) or, with want_p, also P [B,Hq,Tq,Tk].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    g = _group(Hq, Hkv)
    O = np.zeros((B, Tq, Hq, d))
    lse = np.zeros((B, Hq, Tq))
    P_all = np.zeros((B, Hq, Tq, Tk)) if want_p else None
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            for i0 in range(0, Tq, row_block):
                i1 = min(Tq, i0 + row_block)
                kl = _key_limit(i1, Tq, Tk, causal)
                S = scale * (q[b, i0:i1, h, :] @ k[b, :kl, kv, :].T)
                vis = visible_keys(Tq, Tk, causal, np.arange(i0, i1))[:, :kl]
                S = np.where(vis, S, -np.inf)
                m = np.max(S, axis=1, keepdims=True)
                e = np.exp(S - m)
                l = np.sum(e, axis=1, keepdims=True)
                P = e / l
                lse[b, h, i0:i1] = (m + np.log(l))[:, 0]
                O[b, i0:i1, h, :] = P @ v[b, :kl, kv, :]
                if want_p:
                    P_all[b, h, i0:i1, :kl] = P
    if want_p:
        return O, lse, P_all
    return O, lse


def attention_forward_online(q, k, v, scale: float, causal: bool):
    """The same forward by the online softmax that the Hesper pull request's commit log
    describes for FlashAttention.lean (flashAttentionSpec: K and V consumed one position
    at a time, stated equal to the standard scores -> softmax -> apply form).

    Per query row: a running maximum m, a running sum of exponentials l and a running
    weighted sum u of value rows. Each visible key j with score s rescales l and u by
    exp(m_old - m_new) before adding exp(s - m_new) and exp(s - m_new) v_j; at the end
    O = u / l and lse = m + ln l. Plain loops over rows and keys: small cases only.

    Returns (O [B,Tq,Hq,d], lse [B,Hq,Tq]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    g = _group(Hq, Hkv)
    O = np.zeros((B, Tq, Hq, d))
    lse = np.zeros((B, Hq, Tq))
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            for i in range(Tq):
                m, l, u = -np.inf, 0.0, np.zeros(d)
                for j in range(Tk):
                    if causal and j > i + (Tk - Tq):
                        break
                    s = scale * float(q[b, i, h] @ k[b, j, kv])
                    m_new = max(m, s)
                    a = np.exp(m - m_new)     # 0 for the first key (m = -inf)
                    e = np.exp(s - m_new)
                    l = l * a + e
                    u = u * a + e * v[b, j, kv]
                    m = m_new
                O[b, i, h] = u / l
                lse[b, h, i] = m + np.log(l)
    return O, lse


def attention_lse(q, k, scale: float, causal: bool, row_block: int = 1024, q_heads=None):
    """Row log-sum-exp of the scaled scores over visible keys, [B, Hq, Tq].

    With q_heads, only those heads are computed (the rest stay zero).
    """
    q, k = _f64(q), _f64(k)
    B, Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    g = _group(Hq, Hkv)
    lse = np.zeros((B, Hq, Tq))
    heads = range(Hq) if q_heads is None else q_heads
    for b in range(B):
        for h in heads:
            kv = h // g
            for i0 in range(0, Tq, row_block):
                i1 = min(Tq, i0 + row_block)
                kl = _key_limit(i1, Tq, Tk, causal)
                S = scale * (q[b, i0:i1, h, :] @ k[b, :kl, kv, :].T)
                vis = visible_keys(Tq, Tk, causal, np.arange(i0, i1))[:, :kl]
                S = np.where(vis, S, -np.inf)
                m = np.max(S, axis=1, keepdims=True)
                lse[b, h, i0:i1] = (m + np.log(np.sum(np.exp(S - m), axis=1, keepdims=True)))[:, 0]
    return lse


def attention_backward(q, k, v, dout, scale: float, causal: bool, lse=None, P=None,
                       kv_heads=None, row_block: int = 1024, O=None):
    """dQ, dK, dV of the attention output given dO (see the module docstring).

    P (the saved softmax) takes precedence; otherwise P_ij = exp(scale q_i.k_j - lse_i)
    with lse as given (not renormalised); with neither, lse is computed first.
    Entries of a given P at masked (invisible) positions are ignored.

    O: the forward's output [B, Tq, Hq, d], when the caller saved it. Then the row term
    is D_i = dO_i . O_i instead of rowsum(P o dP): with O_i = sum_j P_ij v_j the two are
    equal (sum_j P_ij (dO_i . v_j) = dO_i . sum_j P_ij v_j), so an exact O changes nothing
    and a rounded O enters only through D.

    kv_heads: optional list of kv-heads to compute; then dq holds only the q-heads of
    those groups ([B, Tq, len(kv_heads)*g, d], in group order) and dk, dv only those
    kv-heads ([B, Tk, len(kv_heads), d]).
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    g = _group(Hq, Hkv)
    kvs = list(range(Hkv)) if kv_heads is None else list(kv_heads)
    if P is None and lse is None:
        lse = attention_lse(q, k, scale, causal, row_block,
                            q_heads=[kv * g + j for kv in kvs for j in range(g)])
    dq = np.zeros((B, Tq, len(kvs) * g, d))
    dk = np.zeros((B, Tk, len(kvs), d))
    dv = np.zeros((B, Tk, len(kvs), d))
    for b in range(B):
        for ki, kv in enumerate(kvs):
            for j in range(g):                       # group heads in increasing order
                h = kv * g + j
                for i0 in range(0, Tq, row_block):
                    i1 = min(Tq, i0 + row_block)
                    kl = _key_limit(i1, Tq, Tk, causal)
                    if kl == 0:
                        continue
                    vis = visible_keys(Tq, Tk, causal, np.arange(i0, i1))[:, :kl]
                    kk, vv = k[b, :kl, kv, :], v[b, :kl, kv, :]
                    qi, doi = q[b, i0:i1, h, :], dout[b, i0:i1, h, :]
                    if P is not None:
                        Pb = np.where(vis, _f64(P[b, h, i0:i1, :kl]), 0.0)
                    else:
                        S = scale * (qi @ kk.T)
                        Pb = np.where(vis, np.exp(np.where(vis, S, 0.0) - _f64(lse[b, h, i0:i1])[:, None]), 0.0)
                    dP = doi @ vv.T
                    if O is None:
                        D = np.sum(Pb * dP, axis=1, keepdims=True)
                    else:
                        D = np.sum(doi * _f64(O[b, i0:i1, h, :]), axis=1, keepdims=True)
                    dS = Pb * (dP - D)
                    dq[b, i0:i1, ki * g + j, :] = scale * (dS @ kk)
                    dk[b, :kl, ki, :] += scale * (dS.T @ qi)
                    dv[b, :kl, ki, :] += Pb.T @ doi
    return dq, dk, dv


def softmax_row_dot(P, dP) -> np.ndarray:
    """D_i = sum_j P_ij dP_ij, the row term of softmaxBackward (exposed for checks)."""
    return np.sum(_f64(P) * _f64(dP), axis=-1)
