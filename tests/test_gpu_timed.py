"""attn_bwd_timed (through the binding's events argument) against attn_bwd on the GPU: the
same outputs bit for bit, and the four caller events recorded by the two kernels in order,
on the MFMA path (bf16, d 128, lse given), the flash path (fp32, d 64) and the decode path
(also with keys in one chunk, where the untimed call runs one fused kernel)."""

import ctypes
import os

import numpy as np
import pytest
import torch

import synth
import verified_transformer_backward_amd as vtb
from tests.gpu_helpers import dev, need_gpu, say

pytestmark = pytest.mark.gpu


class _Events:
    """hipEvent_t handles from the HIP runtime torch loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(4):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.ev.append(e.value)

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) == 0
        return out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


CASES = [
    # name, B, Tq, Tk, Hq, Hkv, D, dtype, causal, lse given
    ("mfma_bf16_causal_d128", 2, 192, 192, 4, 2, 128, "bf16", True, True),
    ("flash_f32_causal_d64", 1, 100, 100, 3, 3, 64, "f32", True, False),
    ("decode_f32_gqa4", 2, 1, 300, 8, 2, 128, "f32", False, False),
    # keys in one 64-key chunk: attn_bwd runs one fused kernel, the timed call its two kernels
    ("decode_one_chunk_f32", 2, 1, 64, 8, 2, 128, "f32", False, False),
    ("decode_one_chunk_bf16_causal_lse", 1, 3, 17, 4, 2, 64, "bf16", True, True),
    ("decode_one_chunk_16_rows", 1, 1, 40, 16, 1, 128, "f32", False, False),
    ("decode_one_key", 3, 2, 1, 6, 3, 64, "f32", False, False),
]


@pytest.mark.parametrize("name,B,Tq,Tk,Hq,Hkv,D,dtype,causal,with_lse", CASES)
def test_timed_matches_untimed(name, B, Tq, Tk, Hq, Hkv, D, dtype, causal, with_lse):
    need_gpu()
    say(f"attn_bwd_timed {name}")
    x = synth.attention_inputs(B, Tq, Tk, Hq, Hkv, D, seed=900 + Tk, dtype=dtype)
    t = {n: dev(x[n], dtype) for n in ("q", "k", "v", "dout")}
    sc = 1.0 / np.sqrt(D)
    lse = vtb.attn_fwd_lse(t["q"], t["k"], sc, causal) if with_lse else None
    ref = vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], sc, causal, lse=lse)
    ev = _Events()
    try:
        got = vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], sc, causal, lse=lse, events=ev.ev)
        torch.cuda.synchronize()
        for n, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), f"{name}: {n} differs between attn_bwd_timed and attn_bwd"
        assert ev.hip.hipEventSynchronize(ev.ev[3]) == 0
        first, second, between = ev.ms(0, 1), ev.ms(2, 3), ev.ms(1, 2)
        say(f"  kernels {first * 1e3:.1f} us, {second * 1e3:.1f} us, {between * 1e3:.1f} us between")
        assert first > 0 and second > 0 and between >= 0
        assert first < 1e3 and second < 1e3
    finally:
        ev.close()
