"""Python binding of libvtb, the MI355X (gfx950) attention-layer backward library.

Argument marshalling only: every computation runs in the library's HIP kernels. PyTorch
provides device memory (tensors) and the current HIP stream. There is no fallback: if
libvtb.so is missing or a call fails, an exception is raised.

Entry points (same names as the C ABI in include/vtb.h):
    attn_bwd, attn_fwd, attn_fwd_lse, rope_bwd, rmsnorm_bwd, rope_rmsnorm_res_bwd, linear_bwd,
    layer_bwd, plus the workspace-size queries.
Attention tensors use the [B, T, H, D] layout (any strides, D contiguous).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvtb.so")

VTB_F32, VTB_BF16 = 0, 1
_STATUS = {0: "VTB_OK", 1: "VTB_ERR_ARG", 2: "VTB_ERR_UNSUPPORTED", 3: "VTB_ERR_ALIAS", 4: "VTB_ERR_WORKSPACE", 5: "VTB_ERR_HIP"}

EXPORTS = (
    "vtb_status_string", "vtb_last_error", "vtb_abi_version",
    "attn_bwd_workspace_size", "attn_bwd", "attn_bwd_o", "attn_bwd_timed", "attn_bwd_noalloc", "attn_bwd_noalloc_max_workspace",
    "attn_fwd", "attn_fwd_workspace_size", "attn_fwd_ws", "attn_fwd_lse",
    "rope_bwd", "rmsnorm_bwd", "rope_bwd_ex", "rmsnorm_bwd_ex", "rope_rmsnorm_res_bwd", "linear_bwd", "layernorm_bwd",
    "relu2_mul_bwd",
    "layer_bwd_workspace_size", "layer_bwd", "ffn_bwd_workspace_size", "ffn_bwd",
    "attn_block_bwd_workspace_size", "attn_block_bwd", "rms_attn_block_bwd_workspace_size", "rms_attn_block_bwd",
)


class VtbError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)}: {detail}")


class AttnBwdDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Tq", ctypes.c_int32), ("Tk", ctypes.c_int32), ("D", ctypes.c_int32),
        ("scale", ctypes.c_float), ("causal", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("s_q", ctypes.c_int64 * 3), ("s_k", ctypes.c_int64 * 3), ("s_v", ctypes.c_int64 * 3),
        ("s_do", ctypes.c_int64 * 3), ("s_dq", ctypes.c_int64 * 3), ("s_dk", ctypes.c_int64 * 3),
        ("s_dv", ctypes.c_int64 * 3),
    ]


class LayerBwdCfg(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
        ("scale", ctypes.c_float), ("eps", ctypes.c_float), ("rope_base", ctypes.c_double),
        ("rope_layout", ctypes.c_int32), ("causal", ctypes.c_int32),
    ]


class LayerSaved(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("x", "gamma", "w", "o", "q", "k", "v", "P")]


class FfnBwdCfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("C", ctypes.c_int32), ("F", ctypes.c_int32), ("eps", ctypes.c_float)]


class AttnBlockCfg(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
                ("scale", ctypes.c_float), ("causal", ctypes.c_int32)]


BLOCK_SAVED = ("ln_y", "ln_sig", "w_qkv", "qkv", "P", "ctx", "w_o")


class AttnBlockSaved(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BLOCK_SAVED]


class RmsAttnBlockCfg(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
                ("scale", ctypes.c_float), ("causal", ctypes.c_int32), ("eps", ctypes.c_float),
                ("rope_base", ctypes.c_double), ("rope_layout", ctypes.c_int32)]


RMS_BLOCK_SAVED = ("x", "gamma", "n", "w_qkv", "qkv", "P", "ctx", "w_o")


class RmsAttnBlockSaved(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in RMS_BLOCK_SAVED]


FFN_SAVED = ("x", "gamma1", "xn", "w_gu", "gu", "gamma2", "hn", "w_down")


class FfnSaved(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in FFN_SAVED]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libvtb.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m verified_transformer_backward_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, F64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_size_t
    sig = {
        "vtb_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "vtb_last_error": (ctypes.c_char_p, []),
        "vtb_abi_version": (ctypes.c_int, []),
        "attn_bwd_workspace_size": (SZ, [ctypes.POINTER(AttnBwdDesc)]),
        "attn_bwd": (ctypes.c_int, [ctypes.POINTER(AttnBwdDesc), P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "attn_bwd_timed": (ctypes.c_int, [ctypes.POINTER(AttnBwdDesc), P, P, P, P, P, P, P, P, P, P, SZ, P,
                                          ctypes.POINTER(ctypes.c_void_p), I32]),
        "attn_bwd_o": (ctypes.c_int, [ctypes.POINTER(AttnBwdDesc), P, P, P, P, P, ctypes.POINTER(I64), P, P, P, P, P,
                                      SZ, P]),
        "attn_bwd_noalloc": (ctypes.c_int, [ctypes.POINTER(AttnBwdDesc), P, P, P, P, P, P, P, P, P, P]),
        "attn_bwd_noalloc_max_workspace": (SZ, []),
        "attn_fwd_lse": (ctypes.c_int, [ctypes.POINTER(AttnBwdDesc), P, P, P, P]),
        "attn_fwd": (ctypes.c_int, [ctypes.POINTER(AttnBwdDesc), P, P, P, P, P, P]),
        "attn_fwd_workspace_size": (SZ, [ctypes.POINTER(AttnBwdDesc)]),
        "attn_fwd_ws": (ctypes.c_int, [ctypes.POINTER(AttnBwdDesc), P, P, P, P, P, P, SZ, P]),
        "rope_bwd": (ctypes.c_int, [P, P, I32, I32, I32, I64, P, I32, F64, I32, P]),
        "rmsnorm_bwd": (ctypes.c_int, [P, P, P, P, I32, I32, F32, P]),
        "rope_bwd_ex": (ctypes.c_int, [I32, P, P, I32, I32, I32, I64, P, I32, F64, I32, P]),
        "rmsnorm_bwd_ex": (ctypes.c_int, [I32, P, P, P, P, I32, I32, F32, P]),
        "rope_rmsnorm_res_bwd": (ctypes.c_int, [P, F32, P, P, P, P, I32, I32, I32, I32, F64, I32, F32, P]),
        "linear_bwd": (ctypes.c_int, [P, P, P, P, P, I32, I32, I32, P]),
        "layernorm_bwd": (ctypes.c_int, [I32, P, P, P, P, I32, I32, P]),
        "relu2_mul_bwd": (ctypes.c_int, [I32, P, P, P, P, P, I64, P]),
        "layer_bwd_workspace_size": (SZ, [ctypes.POINTER(LayerBwdCfg)]),
        "layer_bwd": (ctypes.c_int, [ctypes.POINTER(LayerBwdCfg), ctypes.POINTER(LayerSaved), P, P, P, P, P, P, SZ, P]),
        "ffn_bwd_workspace_size": (SZ, [ctypes.POINTER(FfnBwdCfg)]),
        "ffn_bwd": (ctypes.c_int, [ctypes.POINTER(FfnBwdCfg), ctypes.POINTER(FfnSaved), P, P, P, P, P, SZ, P]),
        "attn_block_bwd_workspace_size": (SZ, [ctypes.POINTER(AttnBlockCfg)]),
        "rms_attn_block_bwd_workspace_size": (SZ, [ctypes.POINTER(RmsAttnBlockCfg)]),
        "rms_attn_block_bwd": (ctypes.c_int, [ctypes.POINTER(RmsAttnBlockCfg), ctypes.POINTER(RmsAttnBlockSaved), P, P, P,
                                              P, P, P, SZ, P]),
        "attn_block_bwd": (ctypes.c_int, [ctypes.POINTER(AttnBlockCfg), ctypes.POINTER(AttnBlockSaved), P, P, P, P, P, SZ,
                                          P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    _lib = L
    return L


def _check(status: int, where: str):
    if status != 0:
        raise VtbError(status, where, lib().vtb_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return VTB_F32
    if dt == torch.bfloat16:
        return VTB_BF16
    raise TypeError(f"unsupported dtype {dt} (float32 or bfloat16)")


def _bthd_strides(t: torch.Tensor, name: str):
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, T, H, D]")
    if t.stride(3) != 1:
        raise ValueError(f"{name} must have a contiguous head dimension")
    return (t.stride(0), t.stride(1), t.stride(2))


def _out(t, shape, name: str, device):
    """A caller-given fp32 output, checked for shape, dtype and layout, or a new one."""
    if t is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    if tuple(t.shape) != tuple(shape) or t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous float32 {tuple(shape)}")
    return t


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def make_attn_desc(q, k, scale, causal, out_dtype=None, dout=None, dq=None, dk=None, dv=None, v=None) -> AttnBwdDesc:
    B, Tq, Hq, D = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    d = AttnBwdDesc()
    d.B, d.Hq, d.Hkv, d.Tq, d.Tk, d.D = B, Hq, Hkv, Tq, Tk, D
    d.scale, d.causal = float(scale), int(bool(causal))
    d.in_dtype = _dtype_code(q.dtype)
    d.out_dtype = _dtype_code(out_dtype if out_dtype is not None else q.dtype)
    for field, t, name in (("s_q", q, "q"), ("s_k", k, "k"), ("s_v", v, "v"), ("s_do", dout, "dout"),
                           ("s_dq", dq, "dq"), ("s_dk", dk, "dk"), ("s_dv", dv, "dv")):
        if t is not None:
            getattr(d, field)[:] = _bthd_strides(t, name)
    return d


def attn_bwd_workspace_size(desc: AttnBwdDesc) -> int:
    return int(lib().attn_bwd_workspace_size(ctypes.byref(desc)))


def attn_fwd_workspace_size(desc: AttnBwdDesc) -> int:
    return int(lib().attn_fwd_workspace_size(ctypes.byref(desc)))


def _same_device(t, ref, name: str):
    if t.device != ref.device:
        raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _check_given(t, shape, dtype, ref, name: str):
    """A caller-given [B, T, H, D] output: its shape, dtype, device and a contiguous head dim."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    _same_device(t, ref, name)
    _bthd_strides(t, name)


def attn_bwd(q, k, v, dout, scale: float, causal: bool, lse=None, P=None, out_dtype=None,
             dq=None, dk=None, dv=None, want_dk: bool = True, want_dv: bool = True, workspace=None, stream=None,
             events=None, o=None):
    """dQ, dK, dV of attention (see include/vtb.h). Returns (dq, dk, dv); dk (dv) is None when
    want_dk (want_dv) is false, and the library then skips it.

    o: the forward's saved output [B, Tq, Hq, D] (q's dtype and device, any strides with a
    contiguous head dim); then attn_bwd_o runs, which needs lse and takes no P.

    events: optional sequence of 4 hipEvent_t handles (ints): events[0]/[1] are recorded
    at the start/end of the call's first kernel, events[2]/[3] of its second
    (attn_bwd_timed)."""
    out_dtype = out_dtype or q.dtype
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _bthd_strides(t, n)
    for t, n in ((k, "k"), (v, "v"), (dout, "dout")):
        if t.dtype != q.dtype or t.device != q.device:
            raise TypeError(f"{n} must match q's dtype and device")
    B, Tq, Hq, D = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k {tuple(k.shape)} does not match q {tuple(q.shape)} in batch or head dim")
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"v {tuple(v.shape)} must have k's shape {tuple(k.shape)}")
    if tuple(dout.shape) != tuple(q.shape):
        raise ValueError(f"dout {tuple(dout.shape)} must have q's shape {tuple(q.shape)}")
    if dq is None:
        dq = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _check_given(dq, q.shape, out_dtype, q, "dq")
    if not want_dk:
        dk = None
    elif dk is None:
        dk = torch.empty(k.shape, dtype=out_dtype, device=q.device)
    if not want_dv:
        dv = None
    elif dv is None:
        dv = torch.empty(v.shape, dtype=out_dtype, device=q.device)
    if dk is not None:
        _check_given(dk, k.shape, out_dtype, q, "dk")
    if dv is not None:
        _check_given(dv, v.shape, out_dtype, q, "dv")
    desc = make_attn_desc(q, k, scale, causal, out_dtype, dout, dq, dk, dv, v)
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, Tq):
            raise TypeError(f"lse must be contiguous float32 {(B, Hq, Tq)}")
        _same_device(lse, q, "lse")
    if P is not None:
        if P.dtype != torch.float32 or not P.is_contiguous() or tuple(P.shape) != (B, Hq, Tq, Tk):
            raise TypeError(f"P must be contiguous float32 {(B, Hq, Tq, Tk)}")
        _same_device(P, q, "P")
    if workspace is None:
        workspace = _workspace(attn_bwd_workspace_size(desc), q.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous uint8 tensor")
    else:
        _same_device(workspace, q, "workspace")
    if o is not None:
        if events is not None:
            raise ValueError("events are not taken with a saved o")
        if o.dtype != q.dtype or tuple(o.shape) != tuple(q.shape):
            raise TypeError(f"o must have q's dtype and shape {tuple(q.shape)}")
        _same_device(o, q, "o")
        so = (ctypes.c_int64 * 3)(*_bthd_strides(o, "o"))
        _check(lib().attn_bwd_o(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(o), so, _ptr(lse),
                                _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), _stream(stream)),
               "attn_bwd_o")
        return dq, dk, dv
    args = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(P),
            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), _stream(stream))
    if events is None:
        _check(lib().attn_bwd(*args), "attn_bwd")
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        _check(lib().attn_bwd_timed(*args, arr, len(events)), "attn_bwd_timed")
    return dq, dk, dv


def attn_fwd(q, k, v, scale: float, causal: bool, out_dtype=None, o=None, lse=None, want_lse: bool = True,
             split_kv: bool = True, workspace=None, stream=None):
    """Attention forward (see include/vtb.h): returns (o [B, Tq, Hq, D], lse [B, Hq, Tq] fp32
    or None when want_lse is false and no lse tensor is given). split_kv (default) calls
    attn_fwd_ws, whose decode-shaped problems run split-KV in a workspace (allocated here
    when none is given); split_kv=False calls attn_fwd."""
    for t, n in ((k, "k"), (v, "v")):
        if t.dtype != q.dtype or t.device != q.device:
            raise TypeError(f"{n} must match q's dtype and device")
    out_dtype = out_dtype or q.dtype
    o = torch.empty(q.shape, dtype=out_dtype, device=q.device) if o is None else o
    B, Tq, Hq, _ = q.shape
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    desc = make_attn_desc(q, k, scale, causal, out_dtype=o.dtype, dq=o, v=v)
    if not split_kv:
        _check(lib().attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _stream(stream)),
               "attn_fwd")
        return o, lse
    need = attn_fwd_workspace_size(desc)
    if need == 0:
        _check(1, "attn_fwd_workspace_size")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif workspace.dtype != torch.uint8 or workspace.device != q.device or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous uint8 tensor on q's device")
    _check(lib().attn_fwd_ws(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace),
                             workspace.numel(), _stream(stream)), "attn_fwd_ws")
    return o, lse


def attn_fwd_lse(q, k, scale: float, causal: bool, lse=None, stream=None):
    """Row log-sum-exp [B, Hq, Tq] (fp32) of the scaled scores over visible keys."""
    B, Tq, Hq, _ = q.shape
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device) if lse is None else lse
    desc = make_attn_desc(q, k, scale, causal)
    _check(lib().attn_fwd_lse(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(lse), _stream(stream)), "attn_fwd_lse")
    return lse


def rope_bwd(dy, pos=None, pos0: int = 0, base: float = 10000.0, layout: int = 0, dx=None, stream=None):
    """R(-theta) on every pair of dy [n_tok, n_heads, head_dim] (fp32 or bf16, heads packed);
    bf16 goes through rope_bwd_ex."""
    if dy.dtype not in (torch.float32, torch.bfloat16) or dy.dim() != 3 or dy.stride(2) != 1 or dy.stride(1) != dy.shape[2]:
        raise ValueError("dy must be float32 or bfloat16 [n_tok, n_heads, head_dim] with packed heads")
    dx = torch.empty_like(dy) if dx is None else dx
    if dx.stride() != dy.stride() or dx.dtype != dy.dtype or dx.shape != dy.shape:
        raise ValueError("dx must have dy's shape, dtype and strides")
    if pos is not None and (pos.dtype != torch.int32 or not pos.is_contiguous()):
        raise TypeError("pos must be contiguous int32")
    n, h, d = dy.shape
    args = (_ptr(dy), _ptr(dx), n, h, d, dy.stride(0), _ptr(pos), int(pos0), float(base), int(layout), _stream(stream))
    if dy.dtype == torch.float32:
        _check(lib().rope_bwd(*args), "rope_bwd")
    else:
        _check(lib().rope_bwd_ex(VTB_BF16, *args), "rope_bwd_ex")
    return dx


def rmsnorm_bwd(x, gamma, dy, eps: float = 1e-6, dx=None, stream=None):
    """rmsNormBackward per row of x, dy [rows, n] (fp32 or bf16 contiguous; gamma fp32 [n]);
    bf16 goes through rmsnorm_bwd_ex."""
    if gamma.dtype != torch.float32 or not gamma.is_contiguous() or gamma.shape != (x.shape[-1],):
        raise TypeError("gamma must be contiguous float32 [n]")
    for t, nm in ((x, "x"), (dy, "dy")):
        if t.dtype not in (torch.float32, torch.bfloat16) or t.dtype != x.dtype or not t.is_contiguous() or t.shape != x.shape:
            raise TypeError(f"{nm} must be contiguous float32 or bfloat16, matching x")
    dx = torch.empty_like(x) if dx is None else dx
    if dx.dtype != x.dtype or dx.shape != x.shape or not dx.is_contiguous():
        raise TypeError("dx must be contiguous and match x")
    rows, n = x.shape
    args = (_ptr(x), _ptr(gamma), _ptr(dy), _ptr(dx), rows, n, float(eps), _stream(stream))
    if x.dtype == torch.float32:
        _check(lib().rmsnorm_bwd(*args), "rmsnorm_bwd")
    else:
        _check(lib().rmsnorm_bwd_ex(VTB_BF16, *args), "rmsnorm_bwd_ex")
    return dx


def rope_rmsnorm_res_bwd(dq, x, gamma, dh_out, n_heads: int, head_dim: int, dq_scale: float = 1.0, pos0: int = 0,
                         base: float = 10000.0, layout: int = 0, eps: float = 1e-6, dh_in=None, stream=None):
    """dh_in = dh_out + rmsNormBackward(x, gamma, ropeBackward(dq_scale * dq)) per token row.
    x, dh_out, dh_in: [T, C] with C = n_heads * head_dim; dq: [T, C] or [T, n_heads, head_dim];
    gamma: [C]. All contiguous float32 on one device."""
    C = int(n_heads) * int(head_dim)
    if dh_out.dim() != 2 or dh_out.shape[1] != C:
        raise ValueError(f"dh_out must be [T, {C}] (n_heads * head_dim), got {tuple(dh_out.shape)}")
    T = dh_out.shape[0]
    shapes = {"dq": ((T, C), (T, n_heads, head_dim)), "x": ((T, C),), "gamma": ((C,),), "dh_out": ((T, C),)}
    for t, nm in ((dq, "dq"), (x, "x"), (gamma, "gamma"), (dh_out, "dh_out")):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise TypeError(f"{nm} must be contiguous float32")
        if tuple(t.shape) not in shapes[nm]:
            raise ValueError(f"{nm} must have shape {' or '.join(str(sh) for sh in shapes[nm])}, got {tuple(t.shape)}")
        _same_device(t, dh_out, nm)
    if dh_in is None:
        dh_in = torch.empty_like(dh_out)
    elif dh_in.dtype != torch.float32 or not dh_in.is_contiguous() or tuple(dh_in.shape) != (T, C):
        raise ValueError(f"dh_in must be contiguous float32 {(T, C)}")
    else:
        _same_device(dh_in, dh_out, "dh_in")
    _check(lib().rope_rmsnorm_res_bwd(_ptr(dq), float(dq_scale), _ptr(x), _ptr(gamma), _ptr(dh_out), _ptr(dh_in), T,
                                      n_heads, head_dim, int(pos0), float(base), int(layout), float(eps),
                                      _stream(stream)), "rope_rmsnorm_res_bwd")
    return dh_in


def layernorm_bwd(dy, y, sig, dx=None, stream=None):
    """lnBwd per row of dy, y [rows, n] (fp32 or bf16, contiguous) with the forward's sigma [rows] (fp32)."""
    if dy.dtype != y.dtype or not dy.is_contiguous() or not y.is_contiguous() or dy.shape != y.shape or dy.dim() != 2:
        raise TypeError("dy and y must be contiguous [rows, n] of one dtype")
    if sig.dtype != torch.float32 or not sig.is_contiguous() or sig.shape != (dy.shape[0],):
        raise TypeError("sig must be contiguous float32 [rows]")
    dx = torch.empty_like(dy) if dx is None else dx
    if dx.dtype != dy.dtype or dx.shape != dy.shape or not dx.is_contiguous():
        raise TypeError("dx must be contiguous and match dy")
    rows, n = dy.shape
    _check(lib().layernorm_bwd(_dtype_code(dy.dtype), _ptr(dy), _ptr(y), _ptr(sig), _ptr(dx), rows, n, _stream(stream)),
           "layernorm_bwd")
    return dx


def relu2_mul_bwd(gate, up, dh, dgate=None, dup=None, stream=None):
    """(dgate, dup) of h = ReLU(gate)^2 * up for the upstream dh (same shape and dtype, contiguous)."""
    for t, nm in ((up, "up"), (dh, "dh")):
        if t.dtype != gate.dtype or t.shape != gate.shape or not t.is_contiguous():
            raise TypeError(f"{nm} must be contiguous and match gate")
    if not gate.is_contiguous():
        raise TypeError("gate must be contiguous")
    dgate = torch.empty_like(gate) if dgate is None else dgate
    dup = torch.empty_like(gate) if dup is None else dup
    for t, nm in ((dgate, "dgate"), (dup, "dup")):
        if t.dtype != gate.dtype or t.shape != gate.shape or not t.is_contiguous():
            raise TypeError(f"{nm} must be contiguous and match gate")
    _check(lib().relu2_mul_bwd(_dtype_code(gate.dtype), _ptr(gate), _ptr(up), _ptr(dh), _ptr(dgate), _ptr(dup),
                               gate.numel(), _stream(stream)), "relu2_mul_bwd")
    return dgate, dup


def linear_bwd(x, w, dy, want_dx: bool = True, want_dw: bool = True, dx=None, dw=None, stream=None):
    """dX = dY W^T, dW = X^T dY for Y = X W: x [T, K], w [K, N], dy [T, N], all contiguous
    float32 on one device. Returns (dx [T, K], dw [K, N]); either is None when not wanted."""
    for t, nm in ((x, "x"), (w, "w"), (dy, "dy")):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.dim() != 2:
            raise TypeError(f"{nm} must be a contiguous float32 matrix")
        _same_device(t, x, nm)
    T, K = x.shape
    N = w.shape[1]
    if w.shape[0] != K:
        raise ValueError(f"w {tuple(w.shape)} must be [K, N] with K = {K} (x is {tuple(x.shape)})")
    if tuple(dy.shape) != (T, N):
        raise ValueError(f"dy must be {(T, N)}, got {tuple(dy.shape)}")
    outs = []
    for want, t, shape, nm in ((want_dx, dx, (T, K), "dx"), (want_dw, dw, (K, N), "dw")):
        if not want:
            outs.append(None)
            continue
        if t is None:
            t = torch.empty(shape, dtype=torch.float32, device=x.device)
        elif t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != shape:
            raise ValueError(f"{nm} must be contiguous float32 {shape}")
        else:
            _same_device(t, x, nm)
        outs.append(t)
    dx, dw = outs
    _check(lib().linear_bwd(_ptr(x), _ptr(w), _ptr(dy), _ptr(dx), _ptr(dw), T, K, N, _stream(stream)), "linear_bwd")
    return dx, dw


def make_layer_cfg(T, H, D, scale, eps=1e-6, rope_base=10000.0, rope_layout=0, causal=True) -> LayerBwdCfg:
    c = LayerBwdCfg()
    c.T, c.H, c.D = T, H, D
    c.scale, c.eps, c.rope_base = float(scale), float(eps), float(rope_base)
    c.rope_layout, c.causal = int(rope_layout), int(bool(causal))
    return c


def layer_bwd_workspace_size(cfg: LayerBwdCfg) -> int:
    return int(lib().layer_bwd_workspace_size(ctypes.byref(cfg)))


def layer_bwd(saved: dict, dh_out, scale: float, eps: float = 1e-6, rope_base: float = 10000.0, rope_layout: int = 0,
              causal: bool = True, dh_in=None, dw=None, dk=None, dv=None, workspace=None, stream=None):
    """One layer's backward over its saved tensors (x, gamma, w, o, q, k, v, P); returns
    (dh_in, dw, dk, dv). q, k, v are [T, H, D]; P is [H, T, T]."""
    T, H, D = saved["q"].shape
    for n in ("x", "gamma", "w", "o", "q", "k", "v", "P"):
        t = saved[n]
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise TypeError(f"saved[{n!r}] must be contiguous float32")
    C = H * D
    want = {"x": (T, C), "gamma": (C,), "w": (C, C), "o": (T, C), "q": (T, H, D), "k": (T, H, D), "v": (T, H, D),
            "P": (H, T, T)}
    for n, shp in want.items():
        if tuple(saved[n].shape) != shp:
            raise ValueError(f"saved[{n!r}] has shape {tuple(saved[n].shape)}, expected {shp}")
    if tuple(dh_out.shape) != (T, C):
        raise ValueError(f"dh_out must be {(T, C)}")
    cfg = make_layer_cfg(T, H, D, scale, eps, rope_base, rope_layout, causal)
    sv = LayerSaved(*[saved[n].data_ptr() for n in ("x", "gamma", "w", "o", "q", "k", "v", "P")])
    dev = dh_out.device
    dh_in = _out(dh_in, (T, C), "dh_in", dev)
    dw = _out(dw, (C, C), "dw", dev)
    dk = _out(dk, (T, H, D), "dk", dev)
    dv = _out(dv, (T, H, D), "dv", dev)
    if workspace is None:
        workspace = _workspace(layer_bwd_workspace_size(cfg), dev)
    _check(lib().layer_bwd(ctypes.byref(cfg), ctypes.byref(sv), _ptr(dh_out), _ptr(dh_in), _ptr(dw), _ptr(dk), _ptr(dv),
                           _ptr(workspace), workspace.numel(), _stream(stream)), "layer_bwd")
    return dh_in, dw, dk, dv


def make_ffn_cfg(T, C, F, eps=1e-6) -> FfnBwdCfg:
    c = FfnBwdCfg()
    c.T, c.C, c.F, c.eps = int(T), int(C), int(F), float(eps)
    return c


def ffn_bwd_workspace_size(cfg: FfnBwdCfg) -> int:
    return int(lib().ffn_bwd_workspace_size(ctypes.byref(cfg)))


def ffn_bwd(saved: dict, dout, eps: float = 1e-6, dx=None, dw_gu=None, dw_down=None, workspace=None, stream=None):
    """One FFN block's backward over its saved tensors (x, gamma1, xn, w_gu, gu, gamma2,
    hn, w_down; fp32 contiguous); returns (dx, dw_gu, dw_down)."""
    for n in FFN_SAVED:
        t = saved[n]
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise TypeError(f"saved[{n!r}] must be contiguous float32")
    if dout.dtype != torch.float32 or not dout.is_contiguous():
        raise TypeError("dout must be contiguous float32")
    T, C = saved["x"].shape
    F = saved["w_down"].shape[0]
    want = {"x": (T, C), "gamma1": (C,), "xn": (T, C), "w_gu": (C, 2 * F), "gu": (T, 2 * F), "gamma2": (F,),
            "hn": (T, F), "w_down": (F, C)}
    for n, shp in want.items():
        if tuple(saved[n].shape) != shp:
            raise ValueError(f"saved[{n!r}] has shape {tuple(saved[n].shape)}, expected {shp}")
    if tuple(dout.shape) != (T, C):
        raise ValueError(f"dout must be {(T, C)}")
    cfg = make_ffn_cfg(T, C, F, eps)
    sv = FfnSaved(*[saved[n].data_ptr() for n in FFN_SAVED])
    dx = _out(dx, (T, C), "dx", dout.device)
    dw_gu = _out(dw_gu, (C, 2 * F), "dw_gu", dout.device)
    dw_down = _out(dw_down, (F, C), "dw_down", dout.device)
    need = ffn_bwd_workspace_size(cfg)
    if workspace is None:
        workspace = _workspace(need, dout.device)
    _check(lib().ffn_bwd(ctypes.byref(cfg), ctypes.byref(sv), _ptr(dout), _ptr(dx), _ptr(dw_gu), _ptr(dw_down),
                         _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)), "ffn_bwd")
    return dx, dw_gu, dw_down


def make_block_cfg(B, T, H, D, scale, causal=True) -> AttnBlockCfg:
    c = AttnBlockCfg()
    c.B, c.T, c.H, c.D, c.scale, c.causal = int(B), int(T), int(H), int(D), float(scale), int(bool(causal))
    return c


def attn_block_bwd_workspace_size(cfg: AttnBlockCfg) -> int:
    return int(lib().attn_block_bwd_workspace_size(ctypes.byref(cfg)))


def attn_block_bwd(saved: dict, dx2, B: int, H: int, scale: float, causal: bool = True, dx=None, dw_qkv=None,
                   dw_o=None, workspace=None, stream=None):
    """One attention block's backward over its saved tensors (ln_y, ln_sig, w_qkv, qkv, P,
    ctx, w_o; fp32 contiguous); dx2 is [B T, C]. Returns (dx, dw_qkv, dw_o)."""
    for n in BLOCK_SAVED:
        t = saved[n]
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise TypeError(f"saved[{n!r}] must be contiguous float32")
    if dx2.dtype != torch.float32 or not dx2.is_contiguous():
        raise TypeError("dx2 must be contiguous float32")
    BT, C = dx2.shape
    if BT % B or C % H:
        raise ValueError("dx2 rows must be B * T and its width H * D")
    T = BT // B
    want = {"ln_y": (BT, C), "ln_sig": (BT,), "w_qkv": (C, 3 * C), "qkv": (BT, 3 * C), "P": (B * H, T, T),
            "ctx": (BT, C), "w_o": (C, C)}
    for n, shp in want.items():
        if tuple(saved[n].shape) != shp:
            raise ValueError(f"saved[{n!r}] has shape {tuple(saved[n].shape)}, expected {shp}")
    cfg = make_block_cfg(B, T, H, C // H, scale, causal)
    sv = AttnBlockSaved(*[saved[n].data_ptr() for n in BLOCK_SAVED])
    dx = _out(dx, (BT, C), "dx", dx2.device)
    dw_qkv = _out(dw_qkv, (C, 3 * C), "dw_qkv", dx2.device)
    dw_o = _out(dw_o, (C, C), "dw_o", dx2.device)
    if workspace is None:
        workspace = _workspace(attn_block_bwd_workspace_size(cfg), dx2.device)
    _check(lib().attn_block_bwd(ctypes.byref(cfg), ctypes.byref(sv), _ptr(dx2), _ptr(dx), _ptr(dw_qkv), _ptr(dw_o),
                                _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "attn_block_bwd")
    return dx, dw_qkv, dw_o


def make_rms_block_cfg(B, T, H, D, scale, causal=True, eps=1e-6, rope_base=10000.0, rope_layout=0) -> RmsAttnBlockCfg:
    c = RmsAttnBlockCfg()
    c.B, c.T, c.H, c.D, c.scale, c.causal = int(B), int(T), int(H), int(D), float(scale), int(bool(causal))
    c.eps, c.rope_base, c.rope_layout = float(eps), float(rope_base), int(rope_layout)
    return c


def rms_attn_block_bwd_workspace_size(cfg: RmsAttnBlockCfg) -> int:
    return int(lib().rms_attn_block_bwd_workspace_size(ctypes.byref(cfg)))


def rms_attn_block_bwd(saved: dict, dx2, B: int, H: int, scale: float, causal: bool = True, eps: float = 1e-6,
                       rope_base: float = 10000.0, rope_layout: int = 0, dx=None, dgamma=None, dw_qkv=None, dw_o=None,
                       workspace=None, stream=None):
    """Backward of one Hesper-form attention layer over its saved tensors (x, gamma, n,
    w_qkv, qkv, P, ctx, w_o; fp32 contiguous); dx2 is [B T, C]. Returns (dx, dgamma,
    dw_qkv, dw_o)."""
    for n in RMS_BLOCK_SAVED:
        t = saved[n]
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise TypeError(f"saved[{n!r}] must be contiguous float32")
        _same_device(t, dx2, f"saved[{n!r}]")
    if dx2.dtype != torch.float32 or not dx2.is_contiguous() or dx2.dim() != 2:
        raise TypeError("dx2 must be a contiguous float32 [B T, C] tensor")
    BT, C = dx2.shape
    if BT % B or C % H:
        raise ValueError("dx2 rows must be B * T and its width H * D")
    T = BT // B
    want = {"x": (BT, C), "gamma": (C,), "n": (BT, C), "w_qkv": (C, 3 * C), "qkv": (BT, 3 * C), "P": (B * H, T, T),
            "ctx": (BT, C), "w_o": (C, C)}
    for n, shp in want.items():
        if tuple(saved[n].shape) != shp:
            raise ValueError(f"saved[{n!r}] has shape {tuple(saved[n].shape)}, expected {shp}")
    cfg = make_rms_block_cfg(B, T, H, C // H, scale, causal, eps, rope_base, rope_layout)
    sv = RmsAttnBlockSaved(*[saved[n].data_ptr() for n in RMS_BLOCK_SAVED])
    dx = _out(dx, (BT, C), "dx", dx2.device)
    dgamma = _out(dgamma, (C,), "dgamma", dx2.device)
    dw_qkv = _out(dw_qkv, (C, 3 * C), "dw_qkv", dx2.device)
    dw_o = _out(dw_o, (C, C), "dw_o", dx2.device)
    if workspace is None:
        workspace = _workspace(rms_attn_block_bwd_workspace_size(cfg), dx2.device)
    _check(lib().rms_attn_block_bwd(ctypes.byref(cfg), ctypes.byref(sv), _ptr(dx2), _ptr(dx), _ptr(dgamma), _ptr(dw_qkv),
                                    _ptr(dw_o), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)), "rms_attn_block_bwd")
    return dx, dgamma, dw_qkv, dw_o
