"""C-ABI checks that need no GPU: the library loads, exports every function include/vtb.h
declares, and rejects bad arguments with the documented status before launching."""

import ctypes
import os
import re

import pytest

import verified_transformer_backward_amd as vtb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "vtb.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    names = set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text))
    return sorted(names - {"sizeof", "defined"})


def test_header_declares_the_five_entry_points():
    names = _declared_functions()
    for n in ("attn_bwd", "rope_bwd", "rmsnorm_bwd", "linear_bwd", "layer_bwd"):
        assert n in names


def test_library_exports_every_declared_function():
    L = vtb.lib()
    for n in _declared_functions():
        assert hasattr(L, n), n
    assert set(_declared_functions()) == set(vtb.EXPORTS)


def test_status_strings_and_version():
    L = vtb.lib()
    assert L.vtb_status_string(0) == b"VTB_OK"
    assert L.vtb_status_string(4) == b"VTB_ERR_WORKSPACE"
    assert L.vtb_abi_version() >= 1


# Fake, never-dereferenced device addresses: validation must fail before any launch.
A0, A1, A2, A3, A4, A5, A6, WS = (0x7F0000000000 + i * 0x10000000 for i in range(8))


def _desc(**kw):
    d = vtb.AttnBwdDesc()
    B, Tq, Tk, Hq, Hkv, D = kw.get("B", 1), kw.get("Tq", 8), kw.get("Tk", 8), kw.get("Hq", 2), kw.get("Hkv", 2), kw.get("D", 64)
    d.B, d.Tq, d.Tk, d.Hq, d.Hkv, d.D = B, Tq, Tk, Hq, Hkv, D
    d.scale, d.causal = kw.get("scale", 0.125), kw.get("causal", 1)
    d.in_dtype = d.out_dtype = kw.get("dtype", vtb.VTB_F32)
    for f, H, T in (("s_q", Hq, Tq), ("s_k", Hkv, Tk), ("s_v", Hkv, Tk), ("s_do", Hq, Tq), ("s_dq", Hq, Tq), ("s_dk", Hkv, Tk), ("s_dv", Hkv, Tk)):
        getattr(d, f)[:] = (T * H * D, H * D, D)
    return d


def _call(d, dq=A4, ws=WS, wsb=1 << 30, lse=None):
    return vtb.lib().attn_bwd(ctypes.byref(d), A0, A1, A2, A3, lse, None, dq, A5, A6, ws, wsb, None)


def test_attn_bwd_validation_codes():
    L = vtb.lib()
    assert L.attn_bwd(None, A0, A1, A2, A3, None, None, A4, A5, A6, WS, 1 << 30, None) == 1
    assert _call(_desc(D=96)) == 2
    assert _call(_desc(Hq=3, Hkv=2)) == 1
    assert _call(_desc(Tq=9, Tk=8, causal=1)) == 1
    assert _call(_desc(Tk=0)) == 1
    assert _call(_desc(dtype=7)) == 1
    assert _call(_desc(), dq=A0) == 3                      # dq aliases q
    assert _call(_desc(), ws=None) == 4
    assert _call(_desc(), wsb=16) == 4
    d = _desc()
    d.s_q[1] = 12                                           # stride not a multiple of 8
    assert _call(d) == 2
    assert b"stride" in L.vtb_last_error()


def test_attn_bwd_dk_dv_are_optional():
    # dk, dv NULL = not wanted: validation passes them (and reaches the workspace check,
    # which fails here so that nothing launches); dq NULL is still an argument error
    L = vtb.lib()
    d = _desc()
    assert L.attn_bwd(ctypes.byref(d), A0, A1, A2, A3, None, None, A4, None, None, WS, 16, None) == 4
    assert L.attn_bwd(ctypes.byref(d), A0, A1, A2, A3, None, None, A4, A5, None, WS, 16, None) == 4
    assert L.attn_bwd(ctypes.byref(d), A0, A1, A2, A3, None, None, A4, None, A6, WS, 16, None) == 4
    assert L.attn_bwd(ctypes.byref(d), A0, A1, A2, A3, None, None, None, A5, A6, WS, 1 << 30, None) == 1
    assert L.attn_bwd(ctypes.byref(d), A0, None, A2, A3, None, None, A4, None, None, WS, 1 << 30, None) == 1


def test_attn_bwd_o_validation_codes():
    # a saved O needs lse; o's strides are checked like every other tensor's; o is an input
    L = vtb.lib()
    d = _desc()
    so = (ctypes.c_int64 * 3)(8 * 2 * 64, 2 * 64, 64)
    LSE, O = A6 + 0x1000000, WS + 0x1000000

    def call(o=O, s_o=so, lse=LSE, dq=A4, ws=WS, wsb=1 << 20):
        return L.attn_bwd_o(ctypes.byref(d), A0, A1, A2, A3, o, s_o, lse, dq, A5, A6, ws, wsb, None)

    assert call(o=None) == 1
    assert call(lse=None) == 1
    assert call(s_o=None) == 1
    bad = (ctypes.c_int64 * 3)(8 * 2 * 64, 2 * 64, 60)
    assert call(s_o=bad) == 2
    assert call(o=O + 8) == 2                              # unaligned
    assert call(dq=O) == 3                                 # dq overlaps o
    assert call(ws=O) == 3                                 # workspace overlaps o
    assert call(wsb=16) == 4


def test_attn_workspace_query():
    assert vtb.attn_bwd_workspace_size(_desc(D=96)) == 0
    d = _desc(B=4, Tq=512, Tk=512, Hq=20, Hkv=20, D=128, dtype=vtb.VTB_BF16)
    n = vtb.attn_bwd_workspace_size(d)
    assert n >= 2 * 4 * 20 * 512 * 4            # fp32 row term D and lse, one value per query row


def test_attn_fwd_ws_validation_codes():
    # decode shape (Hq/Hkv * Tq <= 16 rows per kv head): the split-KV forward needs a
    # workspace of one fp32 D-vector and two statistics per (64-key chunk, query row)
    L = vtb.lib()
    d = _desc(B=8, Tq=1, Tk=1024, Hq=20, Hkv=5, D=128, causal=0)
    need = L.attn_fwd_workspace_size(ctypes.byref(d))
    rows, nch = 8 * 20 * 1, 1024 // 64
    assert need >= nch * rows * (128 + 2) * 4
    assert L.attn_fwd_workspace_size(ctypes.byref(_desc(D=96))) == 0
    assert L.attn_fwd_ws(ctypes.byref(d), A0, A1, A2, A4, None, None, 1 << 30, None) == 4       # no workspace
    assert L.attn_fwd_ws(ctypes.byref(d), A0, A1, A2, A4, None, WS, need - 256, None) == 4     # too small
    assert L.attn_fwd_ws(ctypes.byref(d), A0, A1, A2, A4, None, A4, need, None) == 3           # ws overlaps o
    assert L.attn_fwd_ws(ctypes.byref(d), A0, A1, A2, A4, None, A0, need, None) == 3           # ws overlaps q
    assert L.attn_fwd_ws(ctypes.byref(d), A0, A1, A2, A4, None, WS + 8, need, None) == 2       # unaligned
    assert L.attn_fwd_ws(ctypes.byref(_desc(D=96)), A0, A1, A2, A4, None, WS, need, None) == 2
    assert L.attn_fwd_ws(ctypes.byref(d), A0, A1, None, A4, None, WS, need, None) == 1         # v NULL


def test_elementwise_and_linear_validation_codes():
    L = vtb.lib()
    assert L.rope_bwd(A0, A1, 4, 2, 7, 14, None, 0, 10000.0, 0, None) == 1       # odd head_dim
    assert L.rope_bwd(A0, A0 + 8, 4, 2, 8, 16, None, 0, 10000.0, 0, None) == 3    # partial overlap
    assert L.rope_bwd(A0, A1, 4, 2, 8, 16, None, 0, 10000.0, 5, None) == 1        # layout
    assert L.rmsnorm_bwd(A0, A1, A2, A0, 4, 64, 1e-6, None) == 3                  # dx aliases x
    assert L.rmsnorm_bwd(A0, A1, A2, A3, 4, 0, 1e-6, None) == 1
    assert L.linear_bwd(A0, A1, A2, None, None, 4, 4, 4, None) == 1
    assert L.linear_bwd(A0, A1, A2, A0, None, 4, 4, 4, None) == 3
    assert L.rope_rmsnorm_res_bwd(A0, 1.0, A1, A2, A3, A4, 4, 64, 128, 0, 1e4, 0, 1e-6, None) == 2  # row > 4096


def test_layer_validation_codes():
    L = vtb.lib()
    cfg = vtb.make_layer_cfg(8, 2, 96, 0.1)
    sv = vtb.LayerSaved(A0, A1, A2, A3, A4, A5, A6, WS)
    assert L.layer_bwd(ctypes.byref(cfg), ctypes.byref(sv), A0 + 0x1000000, A1 + 0x1000000, A2 + 0x1000000,
                       A3 + 0x1000000, A4 + 0x1000000, WS + 0x1000000, 1 << 30, None) == 2
    cfg = vtb.make_layer_cfg(8, 2, 64, 0.1)
    assert L.layer_bwd(ctypes.byref(cfg), None, A0, A1, A2, A3, A4, WS, 1 << 30, None) == 1
    assert vtb.layer_bwd_workspace_size(cfg) > 0
    # outputs and workspace are written with 16-byte vectors: unaligned ones are refused
    sv = vtb.LayerSaved(A0, A1, A2, A3, A4, A5, A6, WS)
    outs = [A0 + 0x1000000, A1 + 0x1000000, A2 + 0x1000000, A3 + 0x1000000, WS + 0x1000000]
    for i in range(5):
        o = list(outs)
        o[i] += 4
        rc = L.layer_bwd(ctypes.byref(cfg), ctypes.byref(sv), A6 + 0x1000000, o[0], o[1], o[2], o[3], o[4], 1 << 30, None)
        assert rc == 2, (i, rc)
        assert b"aligned" in L.vtb_last_error()


def test_norm_ffn_validation_codes():
    L = vtb.lib()
    assert L.layernorm_bwd(7, A0, A1, A2, A3, 4, 64, None) == 1                    # dtype
    assert L.layernorm_bwd(0, A0, A1, A2, A3, 4, 0, None) == 1                     # n = 0
    assert L.layernorm_bwd(0, A0, A1, A2, A0 + 16, 4, 64, None) == 3               # dx overlaps dy
    assert L.layernorm_bwd(1, A0, A1, A2, A3, 0, 64, None) == 0                    # no rows: nothing to do
    assert L.relu2_mul_bwd(0, A0, A1, A2, A3, A3 + 8, 64, None) == 3               # dgate overlaps dup
    assert L.relu2_mul_bwd(0, A0, A1, A2, A1, A4, 64, None) == 3                   # dgate overlaps up
    assert L.relu2_mul_bwd(0, A0, A1, A2, A3, A4, -1, None) == 1
    assert L.relu2_mul_bwd(0, A0, A1, A2, A3, A4, 0, None) == 0
    cfg = vtb.make_ffn_cfg(8, 64, 96)
    need = vtb.ffn_bwd_workspace_size(cfg)
    assert need > 0
    sv = vtb.FfnSaved(A0, A1, A2, A3, A4, A5, A6, WS)
    out = [WS + 0x1000000 * i for i in range(1, 5)]
    assert L.ffn_bwd(ctypes.byref(cfg), ctypes.byref(sv), out[0], out[1], out[2], out[3], out[3] + 0x800000, 16, None) == 4
    assert L.ffn_bwd(ctypes.byref(cfg), ctypes.byref(sv), out[0], A0, out[2], out[3], out[3] + 0x800000, need, None) == 3
    assert L.ffn_bwd(ctypes.byref(cfg), None, out[0], out[1], out[2], out[3], out[3] + 0x800000, need, None) == 1
    assert L.ffn_bwd(ctypes.byref(cfg), ctypes.byref(sv), out[0], out[1] + 4, out[2], out[3], out[3] + 0x800000, need,
                     None) == 2                                                     # misaligned dx
    bad = vtb.make_ffn_cfg(8, 64, 0)
    assert L.ffn_bwd(ctypes.byref(bad), ctypes.byref(sv), out[0], out[1], out[2], out[3], out[3] + 0x800000, need, None) == 1


def test_attn_block_validation_codes():
    L = vtb.lib()
    cfg = vtb.make_block_cfg(2, 16, 2, 8, 0.35)
    need = vtb.attn_block_bwd_workspace_size(cfg)
    assert need > 0
    sv = vtb.AttnBlockSaved(A0, A1, A2, A3, A4, A5, A6)
    out = [WS + 0x1000000 * i for i in range(1, 5)]
    ok = lambda c=cfg, s=sv, dx2=out[0], dx=out[1], ws=out[3] + 0x800000, wsb=need: L.attn_block_bwd(
        ctypes.byref(c), None if s is None else ctypes.byref(s), dx2, dx, out[2], out[3], ws, wsb, None)
    assert ok(wsb=64) == 4                         # workspace too small
    assert ok(dx=A3) == 3                          # dx overlaps qkv
    assert ok(s=None) == 1
    assert ok(dx=out[1] + 8) == 2                  # misaligned dx
    bad = vtb.make_block_cfg(2, 16, 0, 8, 0.35)
    assert ok(c=bad) == 1


def test_rms_attn_block_validation_codes():
    L = vtb.lib()
    cfg = vtb.make_rms_block_cfg(1, 8, 2, 8, 0.35)
    sv = vtb.RmsAttnBlockSaved(*[A0 + i * 0x1000000 for i in range(8)])
    need = L.rms_attn_block_bwd_workspace_size(ctypes.byref(cfg))
    assert need > 0

    def call(c=cfg, s=sv, dx2=A1 + 0x9000000, dx=A2, dg=A3, dq=A4, do=A5, ws=WS, wsb=need):
        return L.rms_attn_block_bwd(ctypes.byref(c), ctypes.byref(s), dx2, dx, dg, dq, do, ws, wsb, None)

    assert L.rms_attn_block_bwd(None, ctypes.byref(sv), A1, A2, A3, A4, A5, WS, need, None) == 1
    assert call(c=vtb.make_rms_block_cfg(1, 8, 2, 7, 0.35)) == 1            # odd head dim
    assert call(c=vtb.make_rms_block_cfg(1, 8, 2, 8, 0.35, eps=0.0)) == 1    # eps must be positive
    assert call(c=vtb.make_rms_block_cfg(1, 8, 2, 8, 0.35, rope_layout=2)) == 1
    assert call(dg=None) == 1
    assert call(dg=A3 + 4) == 2                                             # unaligned
    assert call(dx=A0) == 3                                                 # dx over the saved x
    assert call(dq=A2) == 3                                                 # two outputs on one buffer
    assert call(wsb=need - 256) == 4


def test_bf16_elementwise_entry_points_validate():
    L = vtb.lib()
    assert L.rope_bwd_ex(5, A0, A1, 4, 2, 8, 16, None, 0, 10000.0, 0, None) == 1        # dtype
    assert L.rope_bwd_ex(1, A0, A0 + 8, 4, 2, 8, 16, None, 0, 10000.0, 0, None) == 3    # partial overlap
    assert L.rope_bwd_ex(1, A0, A1, 0, 2, 8, 16, None, 0, 10000.0, 0, None) == 0        # no tokens
    assert L.rmsnorm_bwd_ex(1, A0, A1, A2, A0, 4, 64, 1e-6, None) == 3                  # dx aliases x
    assert L.rmsnorm_bwd_ex(9, A0, A1, A2, A3, 4, 64, 1e-6, None) == 1


def test_attn_bwd_timed_validation_codes():
    # the events are checked first (four handles needed), then the same validation as attn_bwd
    L = vtb.lib()
    d = _desc()
    args = (ctypes.byref(d), A0, A1, A2, A3, None, None, A4, A5, A6, WS, 1 << 30, None)
    ev = (ctypes.c_void_p * 4)(A0, A1, A2, A3)
    assert L.attn_bwd_timed(*args, None, 4) == 1
    assert L.attn_bwd_timed(*args, ev, 3) == 1
    assert b"4 events" in L.vtb_last_error()
    bad = _desc(D=96)
    assert L.attn_bwd_timed(ctypes.byref(bad), A0, A1, A2, A3, None, None, A4, A5, A6, WS, 1 << 30, None, ev, 4) == 2
    assert L.attn_bwd_timed(ctypes.byref(d), A0, A1, A2, A3, None, None, A0, A5, A6, WS, 1 << 30, None, ev, 4) == 3
