"""GPU parity of attn_bwd_o (the backward with the forward's saved O) against the float64
oracle given the same O: the row term is D_i = dO_i . O_i on both sides."""

import numpy as np
import pytest
import torch

import synth
import verified_transformer_backward_amd as vtb
from oracle import attention as A
from tests.gpu_helpers import TOL, assert_close, dev, host, need_gpu, say

pytestmark = pytest.mark.gpu


def _inputs(B, Tq, Tk, Hq, Hkv, D, dtype, causal, seed):
    x = synth.attention_inputs(B, Tq, Tk, Hq, Hkv, D, seed=seed, dtype=dtype)
    sc = 1.0 / np.sqrt(D)
    O, lse = A.attention_forward(x["q"], x["k"], x["v"], sc, causal)
    # the saved O in the input dtype: exactly these values reach both sides
    O = synth.bf16_round(O) if dtype == "bf16" else O.astype(np.float32)
    return x, sc, O, lse.astype(np.float32)


def _run(x, dtype, sc, causal, O, lse, out_dtype=None, o_layout="bthd"):
    need_gpu()
    t = {n: dev(x[n], dtype) for n in ("q", "k", "v", "dout")}
    o = dev(O, dtype)
    if o_layout == "bhtd":
        o = o.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    od = {None: None, "f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    dq, dk, dv = vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], sc, causal, lse=dev(lse), out_dtype=od, o=o)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv)


def _check(name, got, ref, tol):
    for n, g, r in zip(("dq", "dk", "dv"), got, ref):
        e = assert_close(f"{name}.{n}", g, r, tol)
        say(f"{name}.{n} rel_err={e:.2e}")


CASES = [
    # name, B, Tq, Tk, Hq, Hkv, D, dtype, causal   (path)
    ("bf16_causal_ragged_d128", 2, 200, 200, 3, 3, 128, "bf16", True),        # MFMA
    ("bf16_causal_gqa_TqltTk_d128", 2, 64, 160, 4, 2, 128, "bf16", True),     # MFMA
    ("bf16_noncausal_T96_d128", 1, 96, 96, 2, 2, 128, "bf16", False),         # MFMA
    ("bf16_causal_d64", 2, 100, 100, 2, 1, 64, "bf16", True),                 # flash
    ("f32_causal_ragged_d64", 2, 150, 150, 4, 2, 64, "f32", True),            # flash
    ("f32_noncausal_gqa_TqltTk_d128", 1, 37, 200, 4, 1, 128, "f32", False),   # flash
    ("f32_decode_Tq1", 2, 1, 300, 8, 2, 128, "f32", False),                   # decode: O not read
]


@pytest.mark.parametrize("name,B,Tq,Tk,Hq,Hkv,D,dtype,causal", CASES)
def test_saved_o_cases(name, B, Tq, Tk, Hq, Hkv, D, dtype, causal):
    say(f"attn_bwd_o {name}: B{B} Tq{Tq} Tk{Tk} Hq{Hq} Hkv{Hkv} d{D} {dtype} causal={causal}")
    x, sc, O, lse = _inputs(B, Tq, Tk, Hq, Hkv, D, dtype, causal, seed=900 + Tq + Tk + D)
    ref = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, causal, lse=lse, O=O)
    _check(name, _run(x, dtype, sc, causal, O, lse), ref, TOL[dtype])


def test_saved_o_causal_train_full_size_strided_o():
    say("attn_bwd_o causal B4 H20 T512 d128 bf16, head-major O, fp32 out")
    x = synth.causal_inputs()
    sc = x["scale"]
    O, lse = A.attention_forward(x["q"], x["k"], x["v"], sc, True)
    O = synth.bf16_round(O)
    lse = lse.astype(np.float32)
    ref = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, True, lse=lse, O=O)
    _check("saved_o_train", _run(x, "bf16", sc, True, O, lse, out_dtype="f32", o_layout="bhtd"), ref, TOL["bf16"])


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_saved_o_is_read(dtype, D):
    # O = 0 gives D = 0 (dS = P o dP): the result must follow the O it is given, not the
    # recomputed row term (which the oracle without O would use)
    say(f"attn_bwd_o with O = 0, {dtype} d{D}")
    x, sc, _, lse = _inputs(2, 80, 80, 2, 2, D, dtype, True, seed=990 + D)
    zero = np.zeros_like(x["q"], dtype=np.float32)
    ref = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, True, lse=lse, O=zero)
    other = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, True, lse=lse)
    got = _run(x, dtype, sc, True, zero, lse)
    _check(f"saved_o_zero_{dtype}", got, ref, TOL[dtype])
    assert np.max(np.abs(got[0] - other[0])) > 10 * TOL[dtype] * np.max(np.abs(other[0]))
