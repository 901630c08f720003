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


def _attn(B=1, Tq=5, Tk=6, Hq=4, Hkv=2, D=64, dt=torch.bfloat16):
    q = torch.zeros(B, Tq, Hq, D, dtype=dt)
    k = torch.zeros(B, Tk, Hkv, D, dtype=dt)
    return q, k, torch.zeros_like(k), torch.zeros_like(q)


def test_attn_bwd_rejects_mismatched_tensors():
    q, k, v, do = _attn()
    bad = (ValueError, TypeError)
    with pytest.raises(bad, match="v"):
        vtb.attn_bwd(q, k, torch.zeros(1, 7, 2, 64, dtype=torch.bfloat16), do, 0.1, True)
    with pytest.raises(bad, match="dout"):
        vtb.attn_bwd(q, k, v, torch.zeros(1, 5, 4, 32, dtype=torch.bfloat16), 0.1, True)
    with pytest.raises(bad, match="k"):
        vtb.attn_bwd(q, torch.zeros(2, 6, 2, 64, dtype=torch.bfloat16), v, do, 0.1, True)
    # an output whose dtype differs from out_dtype would be written at the wrong element size
    with pytest.raises(bad, match="dq"):
        vtb.attn_bwd(q, k, v, do, 0.1, True, out_dtype=torch.float32, dq=torch.zeros_like(q))
    with pytest.raises(bad, match="dk"):
        vtb.attn_bwd(q, k, v, do, 0.1, True, dk=torch.zeros(1, 6, 2, 32, dtype=torch.bfloat16))
    with pytest.raises(bad, match="dv"):
        vtb.attn_bwd(q, k, v, do, 0.1, True, out_dtype=torch.float32, dv=torch.zeros(1, 6, 2, 64, dtype=torch.bfloat16))
    with pytest.raises(bad, match="lse"):
        vtb.attn_bwd(q, k, v, do, 0.1, True, lse=torch.zeros(1, 4, 4))
    with pytest.raises(bad, match="P"):
        vtb.attn_bwd(q, k, v, do, 0.1, True, P=torch.zeros(1, 4, 5, 5))
    with pytest.raises(bad, match="head dim"):
        vtb.attn_bwd(q[..., ::2], k[..., ::2], v[..., ::2], do[..., ::2], 0.1, True)
    with pytest.raises(bad, match="workspace"):
        vtb.attn_bwd(q, k, v, do, 0.1, True, workspace=torch.zeros(16, dtype=torch.float32))


def test_linear_bwd_rejects_mismatched_tensors():
    x, w, dy = _f(4, 8), _f(8, 6), _f(4, 6)
    bad = (ValueError, TypeError)
    with pytest.raises(bad, match="w"):
        vtb.linear_bwd(x, _f(7, 6), dy)
    with pytest.raises(bad, match="dy"):
        vtb.linear_bwd(x, w, _f(4, 5))
    with pytest.raises(bad, match="dx"):
        vtb.linear_bwd(x, w, dy, dx=_f(4, 9))
    with pytest.raises(bad, match="dw"):
        vtb.linear_bwd(x, w, dy, dw=_f(6, 8))
    with pytest.raises(bad, match="x"):
        vtb.linear_bwd(torch.zeros(4, 8, dtype=torch.bfloat16), w, dy)


def test_rope_rmsnorm_res_bwd_rejects_mismatched_tensors():
    T, H, D = 3, 2, 8
    C = H * D
    bad = (ValueError, TypeError)
    with pytest.raises(bad, match="dh_out"):
        vtb.rope_rmsnorm_res_bwd(_f(T, C), _f(T, C), _f(C), _f(T, C + 1), H, D)
    with pytest.raises(bad, match="dq"):
        vtb.rope_rmsnorm_res_bwd(_f(T + 1, C), _f(T, C), _f(C), _f(T, C), H, D)
    with pytest.raises(bad, match="x"):
        vtb.rope_rmsnorm_res_bwd(_f(T, C), _f(T, C - 1), _f(C), _f(T, C), H, D)
    with pytest.raises(bad, match="gamma"):
        vtb.rope_rmsnorm_res_bwd(_f(T, C), _f(T, C), _f(C + 2), _f(T, C), H, D)
    with pytest.raises(bad, match="dh_in"):
        vtb.rope_rmsnorm_res_bwd(_f(T, C), _f(T, C), _f(C), _f(T, C), H, D, dh_in=_f(T, C - 1))
