"""GPU parity of attn_block_bwd (through the C ABI) against the float64 oracle's
transformer attention block: small and ragged shapes, several sequences, causal and
not, and the full T 256, 20 x 128 shape in place."""

import numpy as np
import pytest
import torch

import synth
import verified_transformer_backward_amd as vtb
from oracle import block as BK
from tests.gpu_helpers import TOL, assert_close, dev, host, need_gpu, say

pytestmark = pytest.mark.gpu


def _case(B, T, H, d, causal, seed):
    p = synth.block_inputs(B, T, H, d, seed)
    sc = 1.0 / np.sqrt(d)
    _, sv = BK.block_forward(p["xin"], p["w_qkv"], p["w_o"], B, H, sc, causal)
    saved = {k: np.asarray(v, np.float32) for k, v in sv.items()}    # what a forward would store in fp32
    return saved, p["dx2"], sc


# B, T, H, d, causal: one tile, ragged token counts and widths, two sequences, no mask
BLOCK_CASES = [(2, 1, 2, 8, True), (1, 16, 2, 8, True), (2, 37, 3, 12, True), (2, 64, 4, 32, False), (1, 100, 2, 64, True),
               (3, 5, 1, 4, True), (1, 300, 2, 16, True), (1, 500, 1, 128, True), (2, 48, 12, 128, False)]


@pytest.mark.parametrize("B,T,H,d,causal", BLOCK_CASES)
def test_attn_block_bwd_small(B, T, H, d, causal):
    need_gpu()
    say(f"attn_block_bwd B {B} T {T} H {H} d {d} causal {causal}")
    saved, dx2, sc = _case(B, T, H, d, causal, 40 + T)
    ref = BK.block_backward(saved, dx2, B, H, sc, causal)
    got = vtb.attn_block_bwd({k: dev(v) for k, v in saved.items()}, dev(dx2), B, H, sc, causal)
    torch.cuda.synchronize()
    for name, g, r in zip(("dx", "dw_qkv", "dw_o"), got, ref):
        assert_close(name, host(g), r, TOL["f32"])


def test_attn_block_bwd_full_shape_in_place_twice():
    need_gpu()
    say("attn_block_bwd B 1 T 256 H 20 d 128, dx over dx2, two calls on one workspace")
    saved, dx2, sc = _case(1, 256, 20, 128, True, 1009)
    ref = BK.block_backward(saved, dx2, 1, 20, sc, True)
    sv = {k: dev(v) for k, v in saved.items()}
    ws = torch.empty(vtb.attn_block_bwd_workspace_size(vtb.make_block_cfg(1, 256, 20, 128, sc)), dtype=torch.uint8,
                     device="cuda:0")
    for call in range(2):
        g = dev(dx2)
        dx, dwqkv, dwo = vtb.attn_block_bwd(sv, g, 1, 20, sc, True, dx=g, workspace=ws)
        torch.cuda.synchronize()
        assert dx.data_ptr() == g.data_ptr()
        for name, a, r in zip(("dx", "dw_qkv", "dw_o"), (dx, dwqkv, dwo), ref):
            assert_close(f"{name} call {call}", host(a), r, TOL["f32"])
