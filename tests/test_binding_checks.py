"""The Python binding rejects mismatched shapes before anything reaches the library (CPU
only: every case here raises before a call)."""

import pytest
import torch

import verified_transformer_backward_amd as vtb


def _f(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def _ffn_saved(T=4, C=8, F=6):
    return {"x": _f(T, C), "gamma1": _f(C), "xn": _f(T, C), "w_gu": _f(C, 2 * F), "gu": _f(T, 2 * F),
            "gamma2": _f(F), "hn": _f(T, F), "w_down": _f(F, C)}


def test_ffn_bwd_rejects_mismatched_shapes():
    sv = _ffn_saved()
    sv["gu"] = _f(4, 11)
    with pytest.raises(ValueError, match="gu"):
        vtb.ffn_bwd(sv, _f(4, 8))
    with pytest.raises(ValueError, match="dout"):
        vtb.ffn_bwd(_ffn_saved(), _f(5, 8))
    with pytest.raises(ValueError, match="dw_gu"):
        vtb.ffn_bwd(_ffn_saved(), _f(4, 8), dw_gu=_f(8, 6))


def test_attn_block_bwd_rejects_mismatched_shapes():
    B, T, H, D = 2, 3, 2, 4
    C = H * D
    sv = {"ln_y": _f(B * T, C), "ln_sig": _f(B * T), "w_qkv": _f(C, 3 * C), "qkv": _f(B * T, 3 * C),
          "P": _f(H, T, T), "ctx": _f(B * T, C), "w_o": _f(C, C)}
    with pytest.raises(ValueError, match="P"):
        vtb.attn_block_bwd(sv, _f(B * T, C), B, H, 0.5)
    sv["P"] = _f(B * H, T, T)
    with pytest.raises(ValueError, match="dx"):
        vtb.attn_block_bwd(sv, _f(B * T, C), B, H, 0.5, dx=_f(B * T, C + 1))
    with pytest.raises(ValueError, match="rows"):
        vtb.attn_block_bwd(sv, _f(B * T + 1, C), B, H, 0.5)


def test_layer_bwd_rejects_mismatched_shapes():
    T, H, D = 4, 2, 64
    C = H * D
    sv = {"x": _f(T, C), "gamma": _f(C), "w": _f(C, C), "o": _f(T, C), "q": _f(T, H, D), "k": _f(T, H, D),
          "v": _f(T, H, D), "P": _f(H, T, T + 1)}
    with pytest.raises(ValueError, match="P"):
        vtb.layer_bwd(sv, _f(T, C), 0.125)
    sv["P"] = _f(H, T, T)
    with pytest.raises(ValueError, match="dk"):
        vtb.layer_bwd(sv, _f(T, C), 0.125, dk=_f(T, H, D + 1))
