"""GPU parity of attn_fwd (through the C ABI) against the float64 oracle's forward."""

import numpy as np
import pytest
import torch

import synth
import verified_transformer_backward_amd as vtb
from oracle import attention as A
from tests.gpu_helpers import TOL, assert_close, dev, host, need_gpu, say

pytestmark = pytest.mark.gpu


def _fwd(x, dtype, scale, causal, out_dtype=None, want_lse=True, layout="bthd", split_kv=True):
    need_gpu()
    t = {n: dev(x[n], dtype) for n in ("q", "k", "v")}
    if layout == "bhtd":  # same values, head-major storage: strided [B, T, H, D] views
        t = {n: v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for n, v in t.items()}
    od = {None: None, "f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    o, lse = vtb.attn_fwd(t["q"], t["k"], t["v"], scale, causal, out_dtype=od, want_lse=want_lse, split_kv=split_kv)
    torch.cuda.synchronize()
    return host(o), (None if lse is None else host(lse))


def _check(name, got, ref, tol):
    o, lse = got
    e = assert_close(f"{name}.o", o, ref[0], tol)
    say(f"{name}.o rel_err={e:.2e}")
    if lse is not None:
        # lse is an fp32 statistic of exact inputs: judged on the fp32 bar
        e = assert_close(f"{name}.lse", lse, ref[1], TOL["f32"])
        say(f"{name}.lse rel_err={e:.2e}")


CASES = [
    # name, B, Tq, Tk, Hq, Hkv, D, dtype, causal
    ("f32_causal_ragged_d64", 2, 150, 150, 4, 2, 64, "f32", True),
    ("f32_noncausal_gqa_TqltTk_d128", 1, 37, 200, 4, 1, 128, "f32", False),
    ("f32_causal_T1", 2, 1, 1, 2, 2, 128, "f32", True),
    ("bf16_causal_ragged_d128", 2, 200, 200, 3, 3, 128, "bf16", True),
    ("bf16_causal_gqa_TqltTk_d128", 2, 64, 160, 4, 2, 128, "bf16", True),
    ("bf16_noncausal_T96_d128", 1, 96, 96, 2, 2, 128, "bf16", False),
    ("bf16_causal_d64", 2, 100, 100, 2, 1, 64, "bf16", True),
]


@pytest.mark.parametrize("name,B,Tq,Tk,Hq,Hkv,D,dtype,causal", CASES)
def test_forward_cases(name, B, Tq, Tk, Hq, Hkv, D, dtype, causal):
    say(f"attn_fwd {name}: B{B} Tq{Tq} Tk{Tk} Hq{Hq} Hkv{Hkv} d{D} {dtype} causal={causal}")
    x = synth.attention_inputs(B, Tq, Tk, Hq, Hkv, D, seed=500 + Tq + Tk + D, dtype=dtype)
    sc = 1.0 / np.sqrt(D)
    ref = A.attention_forward(x["q"], x["k"], x["v"], sc, causal)
    _check(name, _fwd(x, dtype, sc, causal), ref, TOL[dtype])


def test_forward_out_dtype_layout_and_no_lse():
    say("attn_fwd bf16 in, fp32 out, head-major strides; then without lse")
    x = synth.attention_inputs(2, 130, 130, 4, 2, 128, seed=541, dtype="bf16")
    sc = 1.0 / np.sqrt(128)
    ref = A.attention_forward(x["q"], x["k"], x["v"], sc, True)
    _check("fwd_f32out_bhtd", _fwd(x, "bf16", sc, True, out_dtype="f32", layout="bhtd"), ref, TOL["bf16"])
    o, lse = _fwd(x, "bf16", sc, True, want_lse=False)
    assert lse is None
    assert_close("fwd_nolse.o", o, ref[0], TOL["bf16"])


@pytest.mark.parametrize("split_kv", [True, False])
def test_forward_decode_gqa_full_size(split_kv):
    say(f"attn_fwd decode GQA B8 Tq1 Hq20 Hkv5 Tk1024 d128 fp32 split_kv={split_kv}")
    x = synth.decode_gqa_inputs()
    ref = A.attention_forward(x["q"], x["k"], x["v"], x["scale"], False)
    _check("fwd_decode", _fwd(x, "f32", x["scale"], False, split_kv=split_kv), ref, TOL["f32"])


# Decode shapes ((Hq/Hkv) Tq <= 16 rows per kv head) that attn_fwd_ws runs split-KV over
# 64-key chunks: one key, a ragged last chunk, exactly one chunk, 16 rows, causal rows that
# see few keys, fp32 in / bf16 out, a long cache.
DECODE_CASES = [
    # name, B, Tq, Tk, Hq, Hkv, D, dtype, causal, out_dtype
    ("f32_Tk1_gqa4", 2, 1, 1, 8, 2, 128, "f32", False, None),
    ("f32_ragged_Tk200", 3, 1, 200, 8, 2, 128, "f32", False, None),
    ("f32_causal_Tq4_d64", 2, 4, 130, 8, 2, 64, "f32", True, None),
    ("bf16_causal_Tq2_Tk65", 2, 2, 65, 12, 3, 128, "bf16", True, None),
    ("bf16_mha_Tq16_Tk64", 1, 16, 64, 2, 2, 128, "bf16", True, None),
    ("bf16_causal_TqeqTk3_d64", 1, 3, 3, 4, 1, 64, "bf16", True, None),
    ("f32_in_bf16_out", 2, 1, 300, 8, 4, 128, "f32", False, "bf16"),
    ("f32_long_cache_Tk32768", 1, 1, 32768, 16, 1, 128, "f32", False, None),
]


@pytest.mark.parametrize("name,B,Tq,Tk,Hq,Hkv,D,dtype,causal,out_dtype", DECODE_CASES)
def test_forward_split_kv_decode_cases(name, B, Tq, Tk, Hq, Hkv, D, dtype, causal, out_dtype):
    say(f"attn_fwd split-KV {name}: B{B} Tq{Tq} Tk{Tk} Hq{Hq} Hkv{Hkv} d{D} {dtype} causal={causal} out={out_dtype}")
    x = synth.attention_inputs(B, Tq, Tk, Hq, Hkv, D, seed=700 + Tq + Tk + D + Hq, dtype=dtype)
    sc = 1.0 / np.sqrt(D)
    ref = A.attention_forward(x["q"], x["k"], x["v"], sc, causal)
    tol = TOL["bf16"] if "bf16" in (dtype, out_dtype) else TOL["f32"]
    _check(name, _fwd(x, dtype, sc, causal, out_dtype=out_dtype, split_kv=True), ref, tol)


def test_forward_causal_train_full_size():
    say("attn_fwd causal B4 H20 T512 d128 bf16")
    x = synth.causal_inputs()
    ref = A.attention_forward(x["q"], x["k"], x["v"], x["scale"], True)
    _check("fwd_train", _fwd(x, "bf16", x["scale"], True), ref, TOL["bf16"])


def test_forward_long_causal_sampled_rows():
    need_gpu()
    say("attn_fwd long causal B1 H32 T8192 d128 bf16; oracle on sampled rows")
    x = synth.long_causal_inputs()
    sc = x["scale"]
    o, lse = _fwd(x, "bf16", sc, True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    rng = np.random.default_rng(8192)
    rows = sorted(set([0, 1, 63, 64, 4095, 8191] + list(rng.integers(0, 8192, 10))))
    heads = [0, 17, 31]
    say(f"long causal: GPU done, oracle on rows {rows} of heads {heads}")
    for i in rows:
        # row i sees keys 0 .. i: a one-query problem over the first i + 1 keys
        ro, rl = A.attention_forward(x["q"][:, i:i + 1], x["k"][:, :i + 1], x["v"][:, :i + 1], sc, True)
        assert_close(f"long.o[{i}]", o[:, i, heads], ro[:, 0, heads], TOL["bf16"])
        assert_close(f"long.lse[{i}]", lse[:, heads, i], rl[:, heads, 0], TOL["f32"])
