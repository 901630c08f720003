"""attn_bwd_noalloc (no device allocation; library-held workspace) against attn_bwd with a
caller workspace: bit-identical results through the C ABI, on two calls in a row, the
second with a smaller problem, on the MFMA, flash and decode paths; and the size limit."""

import ctypes

import numpy as np
import pytest
import torch

import synth
import verified_transformer_backward_amd as vtb
from tests.gpu_helpers import dev, need_gpu, say

pytestmark = pytest.mark.gpu


def _noalloc(t, sc, causal, lse, out_dtype):
    L = vtb.lib()
    outs = [torch.empty(t[n].shape, dtype=out_dtype, device=t["q"].device) for n in ("q", "k", "v")]
    desc = vtb.make_attn_desc(t["q"], t["k"], sc, causal, out_dtype, t["dout"], *outs, t["v"])
    P = ctypes.c_void_p
    rc = L.attn_bwd_noalloc(ctypes.byref(desc), P(t["q"].data_ptr()), P(t["k"].data_ptr()), P(t["v"].data_ptr()),
                            P(t["dout"].data_ptr()), None if lse is None else P(lse.data_ptr()), None,
                            P(outs[0].data_ptr()), P(outs[1].data_ptr()), P(outs[2].data_ptr()),
                            P(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, (rc, L.vtb_last_error())
    return outs


CASES = [
    # name, (B, Tq, Tk, Hq, Hkv, D) first call, second (smaller) call, dtype, causal, lse given
    ("bf16_mfma", (2, 256, 256, 4, 2, 128), (1, 130, 130, 2, 1, 128), "bf16", True, True),
    ("f32_flash", (1, 96, 120, 4, 2, 64), (1, 33, 40, 2, 2, 64), "f32", True, False),
    ("f32_decode", (4, 1, 700, 8, 2, 128), (2, 1, 300, 4, 1, 128), "f32", False, False),
    # keys in one chunk: the fused one-launch decode path
    ("f32_decode_one_chunk", (2, 1, 64, 8, 2, 128), (1, 1, 20, 4, 1, 64), "f32", False, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_attn_bwd(case):
    name, big, small, dtype, causal, with_lse = case
    need_gpu()
    from oracle import attention as A

    for call, shape in enumerate((big, small)):
        B, Tq, Tk, Hq, Hkv, D = shape
        say(f"noalloc {name} call {call} shape {shape}")
        x = synth.attention_inputs(B, Tq, Tk, Hq, Hkv, D, dtype, seed=900 + call)
        sc = 1.0 / np.sqrt(D)
        t = {n: dev(x[n], dtype) for n in ("q", "k", "v", "dout")}
        lse = dev(A.attention_lse(x["q"], x["k"], sc, causal).astype(np.float32)) if with_lse else None
        out_dtype = t["q"].dtype
        ref = vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], sc, causal, lse=lse)
        got = _noalloc(t, sc, causal, lse, out_dtype)
        torch.cuda.synchronize()
        for n, g, r in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(g, r), f"{name} call {call} {n} differs from attn_bwd"


def test_noalloc_rejects_problems_beyond_its_array():
    need_gpu()
    L = vtb.lib()
    cap = int(L.attn_bwd_noalloc_max_workspace())
    # lse computed inside: 8 bytes of workspace per query row; ask for more rows than fit
    rows = cap // 8 + 1024
    Hq = 16
    Tq = rows // Hq + 1
    q = torch.empty((1, Tq, Hq, 64), dtype=torch.float32, device="cuda:0")
    desc = vtb.make_attn_desc(q, q, 0.125, True, torch.float32, q, q, q, q, q)
    assert vtb.attn_bwd_workspace_size(desc) > cap
    P = ctypes.c_void_p(q.data_ptr())
    rc = L.attn_bwd_noalloc(ctypes.byref(desc), P, P, P, P, None, None, P, P, P, None)
    assert rc == 4 and b"attn_bwd_noalloc holds at most" in L.vtb_last_error()
