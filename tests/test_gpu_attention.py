"""GPU parity of attn_bwd / attn_fwd_lse (through the C ABI) against the float64 oracle."""

import functools
import zlib

import numpy as np
import pytest
import torch

import synth
import verified_transformer_backward_amd as vtb
from oracle import attention as A
from tests.gpu_helpers import TOL, assert_close, dev, host, need_gpu, say

pytestmark = pytest.mark.gpu


def _run(x, dtype, scale, causal, lse=None, P=None, out_dtype=None, layout="bthd"):
    need_gpu()
    t = {n: dev(x[n], dtype) for n in ("q", "k", "v", "dout")}
    if layout == "bhtd":  # same values, head-major storage: strided [B, T, H, D] views
        t = {n: v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for n, v in t.items()}
    od = {None: None, "f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    lse_t = None if lse is None else dev(lse)
    P_t = None if P is None else dev(P)
    dq, dk, dv = vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], scale, causal, lse=lse_t, P=P_t, out_dtype=od)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv)


def _check(name, got, ref, tol):
    for n, g, r in zip(("dq", "dk", "dv"), got, ref):
        e = assert_close(f"{name}.{n}", g, r, tol)
        say(f"{name}.{n} rel_err={e:.2e}")


def _single_key_term(x, sc):
    """The size one term of dQ or dK would have without the cancellation: |scale dP K|."""
    dp = np.einsum("bqhd,bkhd->bqk", x["dout"].astype(np.float64), x["v"].astype(np.float64))
    return sc * float(np.abs(dp).max()) * float(np.abs(x["k"]).max())


def _check_single_key(name, got, x, sc):
    """One visible key per query: P = 1, so dS = P o (dP - D) = 0 and the mathematics fixes
    dQ = dK = 0 and dV = dO (summed over the group). The kernels form P = exp(S - lse) in
    fp32, which can land one ulp away from 1, so dQ and dK may carry that rounding: they
    must stay within 1e-5 of the uncancelled term |scale dP K| (the 2e-2 bar would allow
    2000 times more). dV must equal dO to the bf16 / fp32 bar."""
    dq, dk, dv = got
    term = _single_key_term(x, sc)
    for n, g in (("dq", dq), ("dk", dk)):
        m = float(np.max(np.abs(g)))
        say(f"{name}.{n} max|.| = {m:.3e} (uncancelled term {term:.3e}, exact zeros: {bool(m == 0.0)})")
        assert np.all(np.isfinite(g)) and m <= 1e-5 * term, f"{name}.{n}: {m:.3e} > 1e-5 x {term:.3e}"


def test_tiny_single_query():
    say("tiny single-query d64 Tk16 fp32, no lse (decode path)")
    t = synth.tiny_inputs()
    got = _run(t, "f32", t["scale"], False)
    ref = A.attention_backward(t["q"], t["k"], t["v"], t["dout"], t["scale"], False)
    _check("tiny", got, ref, TOL["f32"])


def test_decode_gqa_full_size():
    say("decode GQA B8 Hq20 Hkv5 Tk1024 d128 fp32, no lse")
    x = synth.decode_gqa_inputs()
    got = _run(x, "f32", x["scale"], False)
    ref = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], x["scale"], False)
    _check("decode_gqa", got, ref, TOL["f32"])


def test_decode_gqa_with_given_lse():
    say("decode GQA with lse given")
    x = synth.decode_gqa_inputs()
    lse = A.attention_lse(x["q"], x["k"], x["scale"], False)
    got = _run(x, "f32", x["scale"], False, lse=lse.astype(np.float32))
    ref = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], x["scale"], False, lse=lse.astype(np.float32))
    _check("decode_gqa_lse", got, ref, TOL["f32"])


@functools.lru_cache(maxsize=1)
def _causal_train_oracle():
    x = synth.causal_inputs()
    lse = A.attention_lse(x["q"], x["k"], x["scale"], True).astype(np.float32)
    return x, lse, A.attention_backward(x["q"], x["k"], x["v"], x["dout"], x["scale"], True, lse=lse)


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_causal_train_full_size(out_dtype):
    say(f"causal B4 H20 T512 d128 bf16, lse given, out {out_dtype}")
    x, lse, ref = _causal_train_oracle()
    got = _run(x, "bf16", x["scale"], True, lse=lse, out_dtype=out_dtype)
    _check(f"causal_train_{out_dtype}", got, ref, TOL["bf16"])


def test_causal_train_lse_forward():
    need_gpu()
    say("attn_fwd_lse causal B4 H20 T512 d128 bf16")
    x = synth.causal_inputs()
    lse = vtb.attn_fwd_lse(dev(x["q"], "bf16"), dev(x["k"], "bf16"), x["scale"], True)
    torch.cuda.synchronize()
    ref = A.attention_lse(x["q"], x["k"], x["scale"], True)
    # lse is an fp32 statistic of exact inputs: judged on the fp32 bar
    assert_close("lse", host(lse), ref, TOL["f32"])


def test_long_causal_full_size_sampled_heads():
    need_gpu()
    say("long causal B1 H32 T8192 d128 bf16; oracle on heads 0, 17, 31, properties on all")
    x = synth.long_causal_inputs()
    sc = x["scale"]
    heads = [0, 17, 31]
    lse_o = A.attention_lse(x["q"], x["k"], sc, True, q_heads=heads).astype(np.float32)
    t = {n: dev(x[n], "bf16") for n in ("q", "k", "v", "dout")}
    lse = vtb.attn_fwd_lse(t["q"], t["k"], sc, True)     # heads outside the sample use the library's lse
    for h in heads:
        lse[:, h] = torch.from_numpy(lse_o[:, h]).cuda()
    dq, dk, dv = vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], sc, True, lse=lse)
    torch.cuda.synchronize()
    say("long causal: GPU done, oracle on sampled heads")
    ref = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, True, lse=lse_o, kv_heads=heads)
    for n, g, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        e = assert_close(f"long.{n}", host(g[:, :, heads]), r, TOL["bf16"])
        say(f"long.{n} rel_err={e:.2e}")
    # every head: <dQ, Q> = <dK, K> (both equal sum dS o S), outputs finite
    for h in range(32):
        a = float((dq[0, :, h].float() * t["q"][0, :, h].float()).sum())
        b = float((dk[0, :, h].float() * t["k"][0, :, h].float()).sum())
        ref_mag = float(dq[0, :, h].float().abs().sum() * t["q"][0, :, h].float().abs().max())
        assert abs(a - b) <= 2e-2 * ref_mag, (h, a, b)
    assert torch.isfinite(dq.float()).all() and torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()


CASES = [
    # name, B, Tq, Tk, Hq, Hkv, D, dtype, causal
    ("bf16_causal_ragged", 2, 200, 200, 3, 3, 128, "bf16", True),
    ("bf16_causal_gqa_TqltTk_d128", 2, 100, 164, 4, 2, 128, "bf16", True),
    ("bf16_causal_T17_d128", 3, 17, 17, 2, 2, 128, "bf16", True),
    ("bf16_noncausal_Tk1_d128", 1, 20, 1, 2, 2, 128, "bf16", False),
    ("bf16_noncausal_gqa_TqltTk", 1, 77, 300, 8, 2, 128, "bf16", False),
    ("bf16_causal_gqa_TqltTk_d64", 2, 100, 164, 4, 1, 64, "bf16", True),
    ("f32_causal_d64", 1, 96, 96, 2, 2, 64, "f32", True),
    ("f32_noncausal_gqa_d128", 2, 40, 70, 8, 2, 128, "f32", False),
    ("f32_decode_causal_Tq2", 3, 2, 100, 8, 2, 128, "f32", True),
    ("bf16_decode_Tq1_d64", 2, 1, 257, 4, 4, 64, "bf16", False),
    ("bf16_single_key", 1, 1, 1, 2, 2, 64, "bf16", True),
    ("f32_causal_T33", 1, 33, 33, 1, 1, 64, "f32", True),
    # bf16 d 128 MFMA passes: GQA with Tq < Tk on whole blocks, no mask, a 32-row last block
    ("bf16_causal_gqa_Tq64_Tk160", 2, 64, 160, 8, 2, 128, "bf16", True),
    ("bf16_noncausal_T96", 1, 96, 96, 4, 4, 128, "bf16", False),
    ("bf16_causal_T224", 2, 224, 224, 3, 3, 128, "bf16", True),
    # decode path limits: 16 query rows per kv head (the most it takes, its largest LDS use)
    # with a ragged last chunk, in both head dims; more than 16 chunks (several chunk
    # statistics per merging lane, dQ summed without the register prefetch); and 17 rows,
    # one past the decode path, which the general kernels take
    ("f32_decode_R16_causal_Tk300", 2, 2, 300, 16, 2, 128, "f32", True),
    ("bf16_decode_R16_d64", 1, 4, 130, 8, 2, 64, "bf16", False),
    ("f32_decode_Tk1100", 1, 1, 1100, 4, 1, 128, "f32", False),
    ("f32_R17_past_decode", 1, 17, 90, 1, 1, 128, "f32", True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_edge_shapes(case):
    name, B, Tq, Tk, Hq, Hkv, D, dtype, causal = case
    say(f"edge {name}")
    x = synth.attention_inputs(B, Tq, Tk, Hq, Hkv, D, dtype, seed=zlib.crc32(name.encode()) % 100000)
    sc = 1.0 / np.sqrt(D)
    lse = A.attention_lse(x["q"], x["k"], sc, causal).astype(np.float32)
    ref = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, causal, lse=lse)
    got = _run(x, dtype, sc, causal, lse=lse)
    got2 = _run(x, dtype, sc, causal, lse=None)        # lse computed inside
    if Tk == 1:
        for nm, g in ((name, got), (name + "_nolse", got2)):
            _check_single_key(nm, g, x, sc)
            e = assert_close(f"{nm}.dv", g[2], ref[2], TOL[dtype])
            say(f"{nm}.dv rel_err={e:.2e}")
        return
    _check(name, got, ref, TOL[dtype])
    _check(name + "_nolse", got2, ref, TOL[dtype])


def test_consecutive_calls_share_workspace():
    """Two different problems through one workspace, back to back, three times: the row
    term D that the second pass reads must be the current call's."""
    say("bf16 causal B2 T256 H4 d128, two inputs, one workspace")
    sc = 1.0 / np.sqrt(128)
    xs = [synth.attention_inputs(2, 256, 256, 4, 4, 128, "bf16", seed=s) for s in (501, 502)]
    ts = [{n: dev(x[n], "bf16") for n in ("q", "k", "v", "dout")} for x in xs]
    lses = [torch.from_numpy(A.attention_lse(x["q"], x["k"], sc, True).astype(np.float32)).cuda() for x in xs]
    desc = vtb.make_attn_desc(ts[0]["q"], ts[0]["k"], sc, True, torch.bfloat16, ts[0]["dout"], ts[0]["q"], ts[0]["k"],
                              ts[0]["v"], ts[0]["v"])
    ws = torch.empty(vtb.attn_bwd_workspace_size(desc), dtype=torch.uint8, device="cuda:0")
    outs = []
    for rep in range(3):
        for t, lse in zip(ts, lses):
            outs.append(vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], sc, True, lse=lse, workspace=ws))
    torch.cuda.synchronize()
    for i, x in enumerate(xs):
        lse = A.attention_lse(x["q"], x["k"], sc, True).astype(np.float32)
        ref = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, True, lse=lse)
        for rep in range(3):
            _check(f"consecutive_{i}_{rep}", [host(a) for a in outs[2 * rep + i]], ref, TOL["bf16"])


def test_strided_head_major_layout():
    say("bf16 causal, head-major strides")
    x = synth.attention_inputs(2, 130, 130, 4, 4, 128, "bf16", seed=77)
    sc = 1.0 / np.sqrt(128)
    lse = A.attention_lse(x["q"], x["k"], sc, True).astype(np.float32)
    ref = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, True, lse=lse)
    got = _run(x, "bf16", sc, True, lse=lse, layout="bhtd")
    _check("bhtd", got, ref, TOL["bf16"])


def test_saved_softmax_mode_f32():
    say("f32 causal with saved P")
    x = synth.attention_inputs(1, 70, 70, 3, 3, 128, "f32", seed=5)
    sc = 1.0 / np.sqrt(128)
    _, _, P = A.attention_forward(x["q"], x["k"], x["v"], sc, True, want_p=True)
    P32 = P.astype(np.float32)
    ref = A.attention_backward(x["q"], x["k"], x["v"], x["dout"], sc, True, P=P32)
    got = _run(x, "f32", sc, True, P=P32)
    _check("saved_P", got, ref, TOL["f32"])


def test_no_queries_gives_zero_kv_grads():
    need_gpu()
    say("Tq = 0")
    q = torch.zeros((1, 0, 2, 64), device="cuda")
    k = torch.randn((1, 5, 2, 64), device="cuda")
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(k, 7.0)
    vtb.attn_bwd(q, k, k.clone(), q.clone(), 0.125, False, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert float(dk.abs().max()) == 0.0 and float(dv.abs().max()) == 0.0


def test_graph_replay_matches_eager():
    """attn_bwd captured in a HIP graph: every replay, with eager work and synchronisation
    between replays, reproduces the eager result bit for bit."""
    need_gpu()
    say("graph capture: bf16 causal B1 T160 H2 d128, lse given")
    x = synth.attention_inputs(1, 160, 160, 2, 2, 128, "bf16", seed=31)
    sc = 1.0 / np.sqrt(128)
    t = {n: dev(x[n], "bf16") for n in ("q", "k", "v", "dout")}
    lse = vtb.attn_fwd_lse(t["q"], t["k"], sc, True)
    out = {n: torch.empty_like(t[n]) for n in ("q", "k", "v")}
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")

    def call():
        vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], sc, True, lse=lse, dq=out["q"], dk=out["k"], dv=out["v"],
                     workspace=ws, stream=torch.cuda.current_stream())

    call()
    torch.cuda.synchronize()
    ref = {n: v.clone() for n, v in out.items()}
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        call()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cs):
        call()
    for r in range(3):
        for v in out.values():
            v.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for n in out:
            assert torch.equal(out[n], ref[n]), (r, n)
        call()                                      # eager work between replays
        torch.cuda.synchronize()
        say(f"graph replay {r} matches eager")


@pytest.mark.parametrize("case", [("bf16_mfma", 2, 192, 192, 4, 2, 128, "bf16", True, True),
                                  ("f32_flash", 1, 70, 90, 4, 2, 64, "f32", True, False),
                                  ("f32_decode", 2, 1, 300, 8, 2, 128, "f32", False, False),
                                  ("f32_decode_one_chunk", 2, 1, 50, 8, 2, 128, "f32", False, False)],
                         ids=lambda c: c[0])
def test_optional_dk_dv(case):
    """dk and dv are optional: a NULL one is not written and the others are bit-identical to
    the full call's (both NULL skips the key-parallel pass)."""
    name, B, Tq, Tk, Hq, Hkv, D, dtype, causal, with_lse = case
    need_gpu()
    say(f"optional dk/dv {name}")
    x = synth.attention_inputs(B, Tq, Tk, Hq, Hkv, D, dtype, seed=77)
    sc = 1.0 / np.sqrt(D)
    t = {n: dev(x[n], dtype) for n in ("q", "k", "v", "dout")}
    lse = dev(A.attention_lse(x["q"], x["k"], sc, causal).astype(np.float32)) if with_lse else None
    full = vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], sc, causal, lse=lse)
    sentinel = torch.full_like(full[1], 7.0)
    for want_dk, want_dv in ((False, True), (True, False), (False, False)):
        dk0, dv0 = sentinel.clone(), sentinel.clone()
        dq, dk, dv = vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], sc, causal, lse=lse, want_dk=want_dk,
                                  want_dv=want_dv, dk=dk0 if want_dk else None, dv=dv0 if want_dv else None)
        torch.cuda.synchronize()
        assert torch.equal(dq, full[0])
        assert (dk is None) != want_dk and (dv is None) != want_dv
        if want_dk:
            assert torch.equal(dk, full[1])
        if want_dv:
            assert torch.equal(dv, full[2])


@pytest.mark.parametrize("workload,reps", [("causal_train", 5), ("decode_gqa", 5), ("long_causal", 2)])
def test_full_size_repeats_bitwise(workload, reps):
    """The full-size workloads give one result bit for bit, call after call, with other GPU
    work between the calls: every sum runs in a fixed order and nothing uses atomics."""
    need_gpu()
    say(f"{workload}: {reps} calls, each compared bit for bit with the first")
    if workload == "causal_train":
        x, dtype, causal = synth.causal_inputs(), "bf16", True
    elif workload == "decode_gqa":
        x, dtype, causal = synth.decode_gqa_inputs(), "f32", False
    else:
        x, dtype, causal = synth.long_causal_inputs(), "bf16", True
    t = {n: dev(x[n], dtype) for n in ("q", "k", "v", "dout")}
    sc = float(x["scale"])
    lse = vtb.attn_fwd_lse(t["q"], t["k"], sc, causal) if dtype == "bf16" else None
    first = vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], sc, causal, lse=lse)
    torch.cuda.synchronize()
    for r in range(1, reps):
        torch.randn(1 << 22, device="cuda").sum()           # unrelated work on the device between calls
        got = vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], sc, causal, lse=lse)
        torch.cuda.synchronize()
        for n, a, b in zip(("dq", "dk", "dv"), got, first):
            assert torch.equal(a, b), f"{workload} call {r}: {n} differs from the first call"
    say(f"{workload}: {reps} calls identical")
