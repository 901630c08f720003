"""GPU parity of rms_attn_block_bwd (through the C ABI) against the float64 oracle's
Hesper-form attention layer (RMSNorm with gain, Q/K/V projections, RoPE on q and k,
causal attention with the saved softmax, output projection, residual): small and ragged
shapes, several sequences, both RoPE pair layouts, causal and not, and the full
T 256, 20 x 128 shape in place and twice."""

import numpy as np
import pytest
import torch

import synth
import verified_transformer_backward_amd as vtb
from oracle import rms_block as RB
from tests.gpu_helpers import TOL, assert_close, dev, host, need_gpu, say

pytestmark = pytest.mark.gpu

NAMES = ("dx", "dgamma", "dw_qkv", "dw_o")


def _case(B, T, H, d, causal, layout, seed, w_std=None):
    C = H * d
    p = synth.rms_block_inputs(B, T, H, d, seed, w_std=w_std if w_std is not None else 1.0 / np.sqrt(C))
    sc = 1.0 / np.sqrt(d)
    _, sv = RB.rms_block_forward(p["x"], p["gamma"], p["w_qkv"], p["w_o"], B, H, sc, causal, layout=layout)
    saved = {k: np.asarray(v, np.float32) for k, v in sv.items()}    # what a forward would store in fp32
    return saved, p["dx2"], sc


# B, T, H, d, causal, RoPE layout: one token, ragged token counts and widths, several
# sequences, no mask, split-half pairs
CASES = [(2, 1, 2, 8, True, 0), (1, 16, 2, 8, True, 0), (2, 37, 3, 12, True, 1), (2, 64, 4, 32, False, 0),
         (1, 100, 2, 64, True, 1), (3, 5, 1, 4, True, 0), (1, 300, 2, 16, True, 0),
         # the one-kernel dO/dP/dS step with two key tiles per wave (256 < T <= 512), causal and not
         (1, 300, 2, 32, True, 0), (1, 264, 1, 64, False, 1),
         # C = 1536: the output projection's dX comes in two split-K partials, summed per sequence
         (2, 64, 12, 128, True, 0)]


@pytest.mark.parametrize("B,T,H,d,causal,layout", CASES)
def test_rms_attn_block_bwd_small(B, T, H, d, causal, layout):
    need_gpu()
    say(f"rms_attn_block_bwd B {B} T {T} H {H} d {d} causal {causal} layout {layout}")
    saved, dx2, sc = _case(B, T, H, d, causal, layout, 60 + T)
    ref = RB.rms_block_backward(saved, dx2, B, H, sc, causal, layout=layout)
    got = vtb.rms_attn_block_bwd({k: dev(v) for k, v in saved.items()}, dev(dx2), B, H, sc, causal, rope_layout=layout)
    torch.cuda.synchronize()
    for name, g, r in zip(NAMES, got, ref):
        e = assert_close(name, host(g), r, TOL["f32"])
        say(f"  {name} rel_err={e:.2e}")


def test_rms_attn_block_bwd_full_shape_in_place_twice():
    need_gpu()
    say("rms_attn_block_bwd B 1 T 256 H 20 d 128, dx over dx2, two calls on one workspace")
    saved, dx2, sc = _case(1, 256, 20, 128, True, 0, 1010, w_std=0.02)
    ref = RB.rms_block_backward(saved, dx2, 1, 20, sc, True)
    sv = {k: dev(v) for k, v in saved.items()}
    cfg = vtb.make_rms_block_cfg(1, 256, 20, 128, sc)
    ws = torch.empty(vtb.rms_attn_block_bwd_workspace_size(cfg), dtype=torch.uint8, device="cuda:0")
    first = None
    for call in range(2):
        g = dev(dx2)
        out = vtb.rms_attn_block_bwd(sv, g, 1, 20, sc, True, dx=g, workspace=ws)
        torch.cuda.synchronize()
        assert out[0].data_ptr() == g.data_ptr()
        for name, a, r in zip(NAMES, out, ref):
            e = assert_close(f"{name} call {call}", host(a), r, TOL["f32"])
            say(f"  {name} call {call} rel_err={e:.2e}")
        now = [host(a) for a in out]
        if first is None:
            first = now
        else:   # every reduction runs in a fixed order: the second call repeats the first bit for bit
            for name, a, b in zip(NAMES, now, first):
                assert np.array_equal(a, b), f"{name} differs between calls"
