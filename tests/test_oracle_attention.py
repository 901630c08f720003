"""Pins for the oracle's attention backward against facts fixed outside the oracle:
hand-worked fixtures, central differences, torch autograd of an independently written
forward, special cases with closed forms, bilinear identities and structural
equivalences (GQA = MHA on replicated caches, LSE recompute = saved P = fresh softmax)."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import specs, verify
import synth


def _golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "attention_hand.json")))
    ln3 = math.log(3.0)
    ev = lambda v: eval(str(v), {"ln3": ln3}) if isinstance(v, str) else v
    fix = lambda a: np.array([[ev(x) for x in row] if isinstance(row, list) else ev(row) for row in a], dtype=np.float64)
    return [{k: (fix(v) if isinstance(v, list) else v) for k, v in c.items()} for c in g["cases"]]


def test_hand_fixture_single_head_specs(golden_dir):
    for c in _golden(golden_dir):
        q, K, V, do, sc = c["q"], c["K"], c["V"], c["dout"], c["scale"]
        np.testing.assert_allclose(specs.attention_forward(q, K, V, sc), c["out"], atol=1e-15)
        np.testing.assert_allclose(specs.attention_backward_q(q, K, V, sc, do), c["dq"], atol=1e-15)
        np.testing.assert_allclose(specs.attention_backward_k(q, K, V, sc, do), c["dK"], atol=1e-15)
        np.testing.assert_allclose(specs.attention_backward_v(q, K, sc, do), c["dV"], atol=1e-15)


def test_hand_fixture_batched(golden_dir):
    for c in _golden(golden_dir):
        q = c["q"][None, None, None, :]
        K, V = c["K"][None, :, None, :], c["V"][None, :, None, :]
        do = c["dout"][None, None, None, :]
        dq, dk, dv = A.attention_backward(q, K, V, do, c["scale"], causal=False)
        np.testing.assert_allclose(dq[0, 0, 0], c["dq"], atol=1e-15)
        np.testing.assert_allclose(dk[0, :, 0], c["dK"], atol=1e-15)
        np.testing.assert_allclose(dv[0, :, 0], c["dV"], atol=1e-15)


def test_batched_equals_page_single_head_on_tiny_workload():
    t = synth.tiny_inputs()
    q, k, v, do = t["q"], t["k"], t["v"], t["dout"]
    dq, dk, dv = A.attention_backward(q, k, v, do, t["scale"], causal=False)
    q1, K1, V1, d1 = q[0, 0, 0], k[0, :, 0], v[0, :, 0], do[0, 0, 0]
    np.testing.assert_allclose(dq[0, 0, 0], specs.attention_backward_q(q1, K1, V1, t["scale"], d1), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dk[0, :, 0], specs.attention_backward_k(q1, K1, V1, t["scale"], d1), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dv[0, :, 0], specs.attention_backward_v(q1, K1, t["scale"], d1), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("shape", [
    dict(B=1, Tq=3, Tk=4, Hq=2, Hkv=1, d=4, causal=True),
    dict(B=2, Tq=4, Tk=4, Hq=2, Hkv=2, d=3, causal=True),
    dict(B=1, Tq=2, Tk=5, Hq=4, Hkv=2, d=4, causal=False),
    dict(B=1, Tq=1, Tk=6, Hq=4, Hkv=1, d=4, causal=True),
])
def test_attention_fd_page_tolerance(shape):
    res = verify.verify_attention_backward(**shape, seed=2)
    assert all(res.values()), res


def _torch_attention(q, k, v, scale, causal):
    """Forward written independently with torch ops ([B,T,H,d] layout)."""
    B, Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    kk = k.repeat_interleave(g, dim=2)
    vv = v.repeat_interleave(g, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", q, kk) * scale
    if causal:
        i = torch.arange(Tq)[:, None]
        j = torch.arange(Tk)[None, :]
        s = s.masked_fill(j > i + (Tk - Tq), float("-inf"))
    p = torch.softmax(s, dim=-1)
    return torch.einsum("bhij,bjhd->bihd", p, vv)


@pytest.mark.parametrize("causal,Hq,Hkv,Tq,Tk", [(True, 4, 2, 9, 9), (False, 3, 3, 5, 11), (True, 4, 1, 6, 13)])
def test_attention_matches_autograd(causal, Hq, Hkv, Tq, Tk):
    x = synth.attention_inputs(2, Tq, Tk, Hq, Hkv, 8, "f32", seed=21)
    scale = 0.3
    ts = {n: torch.tensor(x[n].astype(np.float64), requires_grad=True) for n in ("q", "k", "v")}
    o = _torch_attention(ts["q"], ts["k"], ts["v"], scale, causal)
    (o * torch.tensor(x["dout"].astype(np.float64))).sum().backward()
    dq, dk, dv = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], scale, causal)
    for ours, ref in ((dq, ts["q"].grad), (dk, ts["k"].grad), (dv, ts["v"].grad)):
        np.testing.assert_allclose(ours, ref.numpy(), rtol=0, atol=1e-12)


def test_single_key_reduces_to_copy():
    # Tk = 1: P = 1, so dS = 0 (dQ = dK = 0) and dV = dO.
    x = synth.attention_inputs(2, 1, 1, 3, 3, 8, seed=4)
    dq, dk, dv = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], 0.5, causal=True)
    assert np.max(np.abs(dq)) == 0.0 and np.max(np.abs(dk)) == 0.0
    np.testing.assert_allclose(dv, x["dout"].astype(np.float64), atol=0)


def test_equal_keys_give_zero_dq():
    x = synth.attention_inputs(1, 4, 6, 2, 2, 8, seed=5)
    k = np.repeat(x["k"][:, :1], 6, axis=1)
    dq, _, _ = A.attention_backward(x["q"], k, x["v"], x["dout"], 0.7, causal=False)
    assert np.max(np.abs(dq)) < 1e-14


def test_causal_first_row_has_zero_dq():
    x = synth.attention_inputs(1, 8, 8, 2, 2, 8, seed=6)
    dq, _, _ = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], 0.4, causal=True)
    assert np.max(np.abs(dq[:, 0])) == 0.0 and np.max(np.abs(dq[:, 1])) > 0


def test_bilinear_identities():
    # <dQ,Q> = <dK,K> = sum dS o S and <dV,V> = <dO,O>, for GQA and causal too.
    x = synth.attention_inputs(2, 12, 12, 4, 2, 16, seed=7)
    sc = 0.25
    dq, dk, dv = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, causal=True)
    O, _ = A.attention_forward(x["q"], x["k"], x["v"], sc, causal=True)
    qd = np.sum(dq * x["q"])
    kd = np.sum(dk * x["k"])
    assert qd == pytest.approx(kd, rel=1e-11)
    assert np.sum(dv * x["v"]) == pytest.approx(np.sum(O * x["dout"]), rel=1e-11)


def test_row_dot_equals_do_dot_o():
    # D_i = rowsum(P o dP) = dO_i . O_i
    x = synth.attention_inputs(1, 10, 10, 2, 2, 8, seed=8)
    sc = 0.35
    O, lse, P = A.attention_forward(x["q"], x["k"], x["v"], sc, causal=True, want_p=True)
    dP = np.einsum("bihd,bjhd->bhij", x["dout"].astype(np.float64), x["v"].astype(np.float64))
    D = A.softmax_row_dot(P, dP)
    np.testing.assert_allclose(D, np.einsum("bihd,bihd->bhi", x["dout"].astype(np.float64), O), rtol=1e-12, atol=1e-13)


def test_saved_o_row_term_matches_the_recomputed_one():
    # With the forward's exact O, D_i = dO_i . O_i equals rowsum(P o dP): the backward is
    # unchanged (GQA, causal, Tq < Tk).
    x = synth.attention_inputs(2, 9, 13, 4, 2, 8, seed=21)
    sc = 0.3
    O, lse = A.attention_forward(x["q"], x["k"], x["v"], sc, causal=True)
    ref = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, causal=True)
    got = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, causal=True, lse=lse, O=O)
    for r, g in zip(ref, got):
        np.testing.assert_allclose(g, r, rtol=1e-11, atol=1e-12)


def test_saved_o_enters_only_through_the_row_term():
    # O = 0 makes D = 0, so dS = P o dP: brute force over every (row, key) pair with
    # dQ_i = scale sum_j P_ij (dO_i . v_j) k_j and dV_j = sum_i P_ij dO_i (dV does not see D).
    x = synth.attention_inputs(1, 5, 5, 2, 1, 4, seed=22)
    sc = 0.5
    _, lse, P = A.attention_forward(x["q"], x["k"], x["v"], sc, causal=True, want_p=True)
    dq, dk, dv = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, causal=True, lse=lse,
                                      O=np.zeros_like(x["q"]))
    q, k, v, do = (x[n].astype(np.float64) for n in ("q", "k", "v", "dout"))
    want_dq = np.zeros_like(dq)
    want_dk = np.zeros_like(dk)
    for h in range(2):
        for i in range(5):
            for j in range(i + 1):
                ds = P[0, h, i, j] * float(do[0, i, h] @ v[0, j, 0])
                want_dq[0, i, h] += sc * ds * k[0, j, 0]
                want_dk[0, j, 0] += sc * ds * q[0, i, h]
    np.testing.assert_allclose(dq, want_dq, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dk, want_dk, rtol=1e-12, atol=1e-14)
    _, _, dv_ref = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, causal=True, lse=lse)
    np.testing.assert_allclose(dv, dv_ref, rtol=1e-12, atol=1e-14)


def test_gqa_equals_mha_on_replicated_caches():
    x = synth.attention_inputs(2, 7, 9, 6, 2, 8, seed=9)
    g = 3
    sc = 0.3
    dq, dk, dv = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, causal=True)
    kr, vr = np.repeat(x["k"], g, axis=2), np.repeat(x["v"], g, axis=2)
    dq2, dk2, dv2 = A.attention_backward(x["q"], kr, vr, x["dout"], sc, causal=True)
    np.testing.assert_allclose(dq, dq2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dk, dk2.reshape(2, 9, 2, g, 8).sum(3), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(2, 9, 2, g, 8).sum(3), rtol=1e-12, atol=1e-13)


def test_lse_recompute_equals_saved_p_equals_fresh_softmax():
    x = synth.attention_inputs(1, 9, 12, 4, 2, 8, seed=10)
    sc = 0.3
    _, lse, P = A.attention_forward(x["q"], x["k"], x["v"], sc, causal=True, want_p=True)
    r0 = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, True)
    r1 = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, True, lse=lse)
    r2 = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, True, P=P)
    for a, b, c in zip(r0, r1, r2):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(a, c, rtol=1e-12, atol=1e-14)


def test_lse_matches_logsumexp():
    x = synth.attention_inputs(1, 5, 8, 2, 1, 4, seed=12)
    sc = 0.9
    lse = A.attention_lse(x["q"], x["k"], sc, causal=True)
    q, k = x["q"].astype(np.float64), x["k"].astype(np.float64)
    for h in range(2):
        for i in range(5):
            s = [sc * np.dot(q[0, i, h], k[0, j, 0]) for j in range(i + 3 + 1)]
            assert lse[0, h, i] == pytest.approx(math.log(sum(math.exp(v) for v in s)), rel=1e-13)


def test_row_blocking_changes_nothing():
    x = synth.attention_inputs(1, 37, 41, 2, 1, 8, seed=13)
    a = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], 0.3, True, row_block=1024)
    b = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], 0.3, True, row_block=8)
    for u, w in zip(a, b):
        np.testing.assert_allclose(u, w, rtol=1e-13, atol=1e-14)


def test_kv_head_subset_matches_full():
    x = synth.attention_inputs(1, 6, 6, 4, 2, 8, seed=14)
    dq, dk, dv = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], 0.3, True)
    sq, sk, sv = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], 0.3, True, kv_heads=[1])
    np.testing.assert_allclose(sq, dq[:, :, 2:4], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(sk[:, :, 0], dk[:, :, 1], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(sv[:, :, 0], dv[:, :, 1], rtol=1e-13, atol=1e-15)


def test_bottom_right_causal_alignment():
    # With Tq < Tk the last query sees every key; the first sees Tk - Tq + 1 keys.
    vis = A.visible_keys(3, 7, True)
    assert vis[2].all() and vis[0].sum() == 5
    assert np.array_equal(A.visible_keys(4, 4, True), np.tril(np.ones((4, 4), bool)))


# ---- forward by online softmax (the FlashAttention.lean entry of the commit log)

@pytest.mark.parametrize("causal,Hq,Hkv,Tq,Tk", [(True, 2, 2, 7, 7), (True, 4, 2, 3, 9), (False, 2, 1, 5, 6)])
def test_online_forward_equals_standard(causal, Hq, Hkv, Tq, Tk):
    # flash == standard, the equivalence the commit log states; the standard form is
    # pinned by the hand fixtures, central differences and autograd above
    x = synth.attention_inputs(2, Tq, Tk, Hq, Hkv, 8, seed=31 + Tq)
    O1, l1 = A.attention_forward(x["q"], x["k"], x["v"], 0.4, causal)
    O2, l2 = A.attention_forward_online(x["q"], x["k"], x["v"], 0.4, causal)
    np.testing.assert_allclose(O2, O1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("fwd", [A.attention_forward, A.attention_forward_online])
def test_forward_zero_keys_average_visible_values(fwd):
    # all scores 0: P uniform over the visible keys, O_i = mean of visible v_j, lse = ln(count)
    x = synth.attention_inputs(1, 5, 8, 2, 2, 4, seed=32)
    k = np.zeros_like(x["k"])
    O, lse = fwd(x["q"], k, x["v"], 0.9, True)
    v = x["v"].astype(np.float64)
    for i in range(5):
        n = i + 3 + 1   # keys 0 .. i + (8 - 5)
        np.testing.assert_allclose(O[0, i], v[0, :n].mean(axis=0), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[0, :, i], math.log(n), rtol=1e-14)


@pytest.mark.parametrize("fwd", [A.attention_forward, A.attention_forward_online])
def test_forward_single_key_copies_value(fwd):
    # Tk = 1: P = 1, O = v_0, lse = the one scaled score
    x = synth.attention_inputs(1, 1, 1, 3, 1, 8, seed=33)
    O, lse = fwd(x["q"], x["k"], x["v"], 0.3, True)
    q, k, v = (x[n].astype(np.float64) for n in ("q", "k", "v"))
    np.testing.assert_allclose(O[0, 0], np.repeat(v[0, 0], 3, axis=0), rtol=0, atol=0)
    np.testing.assert_allclose(lse[0, :, 0], 0.3 * q[0, 0] @ k[0, 0, 0], rtol=1e-15)


# Planted mistakes, each in a copy of the oracle's online forward built from its source on
# the CPU: dropping the rescale of the value sum, of the exponential sum, or the maximum in
# lse must each break the equality with the standard form.
_ONLINE_MISTAKES = {
    "no_value_rescale": ("u = u * a + e * v[b, j, kv]", "u = u + e * v[b, j, kv]"),
    "no_sum_rescale": ("l = l * a + e", "l = l + e"),
    "lse_without_max": ("lse[b, h, i] = m + np.log(l)", "lse[b, h, i] = np.log(l)"),
}


def _planted_online_forward(mistake):
    import inspect
    import textwrap

    src = textwrap.dedent(inspect.getsource(A.attention_forward_online))
    old, new = _ONLINE_MISTAKES[mistake]
    assert src.count(old) == 1, mistake
    ns = dict(vars(A))
    exec(compile(src.replace(old, new), "<planted>", "exec"), ns)
    return ns["attention_forward_online"]


@pytest.mark.parametrize("mistake", sorted(_ONLINE_MISTAKES))
def test_online_forward_planted_mistakes_fail(mistake):
    x = synth.attention_inputs(2, 7, 7, 2, 2, 8, seed=38)
    O1, l1 = A.attention_forward(x["q"], x["k"], x["v"], 0.4, True)
    O2, l2 = _planted_online_forward(mistake)(x["q"], x["k"], x["v"], 0.4, True)
    assert not (np.allclose(O2, O1, rtol=1e-6, atol=1e-8) and np.allclose(l2, l1, rtol=1e-6, atol=1e-8))


def test_online_forward_large_scores_stay_finite():
    # scores far beyond exp's range: the running maximum keeps every term finite
    x = synth.attention_inputs(1, 4, 4, 1, 1, 8, seed=34)
    q = x["q"].astype(np.float64) * 400.0
    O1, l1 = A.attention_forward(q, x["k"], x["v"], 1.0, True)
    O2, l2 = A.attention_forward_online(q, x["k"], x["v"], 1.0, True)
    assert np.all(np.isfinite(O2)) and np.all(np.isfinite(l2))
    np.testing.assert_allclose(O2, O1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=1e-12)
