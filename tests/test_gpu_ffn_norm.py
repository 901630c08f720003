"""GPU parity of layernorm_bwd, relu2_mul_bwd and ffn_bwd (through the C ABI) against the
float64 oracle: fp32 and bf16 storage, vector and any-width kernels, ragged and
misaligned inputs, degenerate sizes and the full FFN shape (T 256, C 2560, F 6912)."""

import numpy as np
import pytest
import torch

import synth
import verified_transformer_backward_amd as vtb
from oracle import norm_ffn as NF
from tests.gpu_helpers import TOL, assert_close, dev, host, need_gpu, say

pytestmark = pytest.mark.gpu


def _store(a, dtype):
    """Round float64 values to the storage precision (fp32, then bf16 RNE for bf16)."""
    a = np.asarray(a, np.float32)
    return synth.bf16_round(a) if dtype == "bf16" else a


def _misaligned(t):
    """A copy of t whose data starts 2 bytes (bf16) or 4 bytes (fp32) past a 16-byte boundary."""
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    out = buf[1:].view(t.shape)
    out.copy_(t)
    return out


# rows, n: vector kernel with 1..4 vectors per thread, widths that are not a multiple of
# the vector, rows wider than the vector path, a single-element row
LN_CASES = [("f32", 3, 64), ("f32", 17, 2560), ("f32", 5, 4096), ("f32", 4, 100), ("f32", 6, 101), ("f32", 2, 5000),
            ("f32", 3, 1), ("bf16", 7, 2560), ("bf16", 3, 8192), ("bf16", 2, 10000), ("bf16", 5, 36)]


@pytest.mark.parametrize("dtype,rows,n", LN_CASES)
def test_layernorm_bwd_shapes(dtype, rows, n):
    need_gpu()
    say(f"layernorm_bwd {dtype} rows {rows} n {n}")
    inp = synth.layernorm_inputs(rows, n, dtype, seed=rows * 7919 + n)
    y64, sig64 = NF.layernorm_forward(inp["x"])
    y, sig = _store(y64, dtype), sig64.astype(np.float32)
    out = vtb.layernorm_bwd(dev(inp["dy"], dtype), dev(y, dtype), dev(sig))
    torch.cuda.synchronize()
    assert_close("layernorm dx", host(out), NF.layernorm_backward(inp["dy"], y, sig), TOL[dtype])


def test_layernorm_bwd_full_shape_and_misaligned():
    need_gpu()
    say("layernorm_bwd f32 7680 x 2560 (the bench shape), then misaligned operands")
    inp = synth.layernorm_inputs(7680, 2560, "f32")
    y64, sig64 = NF.layernorm_forward(inp["x"])
    y, sig = _store(y64, "f32"), sig64.astype(np.float32)
    ref = NF.layernorm_backward(inp["dy"], y, sig)
    dy_d, y_d, sig_d = dev(inp["dy"]), dev(y), dev(sig)
    out = vtb.layernorm_bwd(dy_d, y_d, sig_d)
    torch.cuda.synchronize()
    assert_close("layernorm dx full", host(out), ref, TOL["f32"])
    out2 = vtb.layernorm_bwd(_misaligned(dy_d[:64]), _misaligned(y_d[:64]), sig_d[:64].clone())
    torch.cuda.synchronize()
    assert_close("layernorm dx misaligned", host(out2), ref[:64], TOL["f32"])


def test_layernorm_bwd_row_sums_vanish():
    # mean(y) = 0 and mean(y^2) = 1 make every dx row sum to zero (a property of any size)
    need_gpu()
    say("layernorm_bwd row sums, 64 x 2560")
    inp = synth.layernorm_inputs(64, 2560, "f32", seed=5)
    y64, sig64 = NF.layernorm_forward(inp["x"])
    out = host(vtb.layernorm_bwd(dev(inp["dy"]), dev(y64), dev(sig64.astype(np.float32))))
    scale = np.abs(out).sum(axis=1)
    assert np.all(np.abs(out.sum(axis=1)) <= 1e-5 * scale)


RELU_CASES = [("f32", 1), ("f32", 7), ("f32", 1000), ("f32", 4099), ("f32", 1 << 21), ("bf16", 5), ("bf16", 4099),
              ("bf16", 1 << 21)]


@pytest.mark.parametrize("dtype,n", RELU_CASES)
def test_relu2_mul_bwd_sizes(dtype, n):
    need_gpu()
    say(f"relu2_mul_bwd {dtype} n {n}")
    inp = synth.relu2_inputs(n, dtype, seed=n)
    g, u, d = (dev(inp[k], dtype) for k in ("gate", "up", "dh"))
    dg, du = vtb.relu2_mul_bwd(g, u, d)
    torch.cuda.synchronize()
    rg, ru = NF.relu2_mul_backward(inp["gate"], inp["up"], inp["dh"])
    assert_close("dgate", host(dg), rg, TOL[dtype])
    assert_close("dup", host(du), ru, TOL[dtype])
    # closed gates give exact zeros on both outputs
    closed = inp["gate"] <= 0
    assert np.all(host(dg)[closed] == 0) and np.all(host(du)[closed] == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_relu2_mul_bwd_misaligned(dtype):
    need_gpu()
    say(f"relu2_mul_bwd {dtype} misaligned, n 3001")
    inp = synth.relu2_inputs(3001, dtype, seed=9)
    g, u, d = (_misaligned(dev(inp[k], dtype)) for k in ("gate", "up", "dh"))
    dg, du = vtb.relu2_mul_bwd(g, u, d, dgate=_misaligned(torch.empty_like(g)), dup=_misaligned(torch.empty_like(g)))
    torch.cuda.synchronize()
    rg, ru = NF.relu2_mul_backward(inp["gate"], inp["up"], inp["dh"])
    assert_close("dgate", host(dg), rg, TOL[dtype])
    assert_close("dup", host(du), ru, TOL[dtype])


def test_relu2_mul_bwd_empty():
    need_gpu()
    e = torch.empty(0, device="cuda:0")
    dg, du = vtb.relu2_mul_bwd(e, e, e)
    assert dg.numel() == 0 and du.numel() == 0


def _ffn_case(T, C, F, seed):
    p = synth.ffn_inputs(T, C, F, seed)
    _, sv = NF.ffn_forward(p["x"], p["gamma1"], p["w_gu"], p["gamma2"], p["w_down"])
    saved = {k: np.asarray(v, np.float32) for k, v in sv.items()}   # what a forward would store in fp32
    return saved, p["dout"]


# T, C, F: one tile, ragged tiles (widths not multiples of 4 or of the 64-wide tiles),
# and sub-norm rows on both the vector and the any-width kernels
FFN_CASES = [(1, 64, 96, 20), (16, 64, 96, 21), (37, 200, 300, 22), (50, 130, 75, 23), (64, 512, 8200, 24)]


@pytest.mark.parametrize("T,C,F,seed", FFN_CASES)
def test_ffn_bwd_small(T, C, F, seed):
    need_gpu()
    say(f"ffn_bwd T {T} C {C} F {F}")
    saved, dout = _ffn_case(T, C, F, seed)
    ref = NF.ffn_backward(saved, dout)
    got = vtb.ffn_bwd({k: dev(v) for k, v in saved.items()}, dev(dout))
    torch.cuda.synchronize()
    for name, g, r in zip(("dx", "dw_gu", "dw_down"), got, ref):
        assert_close(name, host(g), r, TOL["f32"])


def test_ffn_bwd_full_shape_in_place_and_repeat():
    # the bench shape; dx written over dout, then a second call on the same workspace
    need_gpu()
    say("ffn_bwd T 256 C 2560 F 6912, in place, two calls")
    saved, dout = _ffn_case(256, 2560, 6912, 1008)
    ref = NF.ffn_backward(saved, dout)
    sv = {k: dev(v) for k, v in saved.items()}
    ws = torch.empty(vtb.ffn_bwd_workspace_size(vtb.make_ffn_cfg(256, 2560, 6912)), dtype=torch.uint8, device="cuda:0")
    for call in range(2):
        g = dev(dout)
        dx, dwgu, dwd = vtb.ffn_bwd(sv, g, dx=g, workspace=ws)
        torch.cuda.synchronize()
        assert dx.data_ptr() == g.data_ptr()
        for name, a, r in zip(("dx", "dw_gu", "dw_down"), (dx, dwgu, dwd), ref):
            assert_close(f"{name} call {call}", host(a), r, TOL["f32"])
