"""Seeded generators for the five attention-backward workloads and for test shapes.

Conventions (fixed so every consumer sees the same numbers):
  * numpy ``default_rng`` (PCG64); draws are made in float64, rounded to float32, then
    to bf16 (round-to-nearest-even) where a workload stores bf16.
  * Attention tensors use the [B, T, H, d] layout (d contiguous, heads strided inside a
    token row), the natural BT x C activation layout of the transformer.js page.
  * Draw order within one seed: q, k, v, dout, then workload-specific tensors.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


# ----------------------------------------------------------------------------- rounding

def bf16_round(x) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(x.shape)


def bf16_bits(x) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact (int16 patterns)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("bf16_bits: values are not bf16-representable; round first")
    return (u >> 16).astype(np.uint16).view(np.int16).reshape(x.shape)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x = x64.astype(np.float32)
    if dtype == "bf16":
        return bf16_round(x)
    if dtype != "f32":
        raise ValueError(f"unknown storage dtype {dtype!r}")
    return x


def normal(rng: np.random.Generator, shape, std: float = 1.0, dtype: str = "f32") -> np.ndarray:
    return _store(rng.standard_normal(size=shape) * std, dtype)


def uniform(rng: np.random.Generator, shape, lo: float, hi: float, dtype: str = "f32") -> np.ndarray:
    return _store(rng.uniform(lo, hi, size=shape), dtype)


# ----------------------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Workload:
    name: str
    what: str
    sizes: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload(
        "tiny",
        "single-head single-query attention backward q[64], K,V[16x64], scale 1/8; "
        "RoPE backward on 32 pairs at pos 5; RMSNorm backward n=64",
        dict(B=1, Tq=1, Tk=16, Hq=1, Hkv=1, d=64, dtype="f32", seed=1001),
    ),
    "decode_gqa": Workload(
        "decode_gqa",
        "decode-shaped GQA attention backward: 8 sequences x 1 query, 20 q-heads on 5 kv-heads, "
        "d 128, KV length 1024, fp32",
        dict(B=8, Tq=1, Tk=1024, Hq=20, Hkv=5, d=128, dtype="f32", seed=1002),
    ),
    "causal_train": Workload(
        "causal_train",
        "causal MHA attention backward B4 H20 T512 d128, bf16 in, fp32 accumulation",
        dict(B=4, Tq=512, Tk=512, Hq=20, Hkv=20, d=128, dtype="bf16", seed=1003),
    ),
    "layer_chain": Workload(
        "layer_chain",
        "30-layer reverse backward chain: T256, hidden 2560 = 20 heads x d128, fp32",
        dict(L=30, T=256, H=20, d=128, dtype="f32", seed=1004),
    ),
    "long_causal": Workload(
        "long_causal",
        "long-context causal attention backward B1 H32 T8192 d128, bf16 in",
        dict(B=1, Tq=8192, Tk=8192, Hq=32, Hkv=32, d=128, dtype="bf16", seed=1005),
    ),
}


def attention_inputs(B, Tq, Tk, Hq, Hkv, d, dtype="f32", seed=0):
    """q, k, v, dout ~ N(0, 1) in [B, T, H, d] layout, in that draw order."""
    rng = np.random.default_rng(seed)
    q = normal(rng, (B, Tq, Hq, d), dtype=dtype)
    k = normal(rng, (B, Tk, Hkv, d), dtype=dtype)
    v = normal(rng, (B, Tk, Hkv, d), dtype=dtype)
    dout = normal(rng, (B, Tq, Hq, d), dtype=dtype)
    return dict(q=q, k=k, v=v, dout=dout)


def tiny_inputs():
    """The single-head, single-query case plus the RoPE and RMSNorm vectors (all fp32)."""
    s = WORKLOADS["tiny"].sizes
    rng = np.random.default_rng(s["seed"])
    out = dict(
        q=normal(rng, (1, 1, 1, 64)),
        k=normal(rng, (1, 16, 1, 64)),
        v=normal(rng, (1, 16, 1, 64)),
        dout=normal(rng, (1, 1, 1, 64)),
    )
    out["scale"] = 1.0 / 8.0
    out["rope_dy"] = normal(rng, (1, 1, 64))      # [tokens, heads, head_dim]: 32 pairs
    out["rope_pos"] = 5
    out["rope_base"] = 10000.0
    out["rms_x"] = normal(rng, (1, 64))
    out["rms_dy"] = normal(rng, (1, 64))
    out["rms_gamma"] = uniform(rng, (64,), 0.5, 1.5)
    out["rms_eps"] = 1e-6
    return out


def decode_gqa_inputs():
    s = WORKLOADS["decode_gqa"].sizes
    out = attention_inputs(s["B"], s["Tq"], s["Tk"], s["Hq"], s["Hkv"], s["d"], "f32", s["seed"])
    out["scale"] = 1.0 / np.sqrt(128.0)
    return out


def causal_inputs(B=4, T=512, H=20, d=128, dtype="bf16", seed=1003):
    out = attention_inputs(B, T, T, H, H, d, dtype, seed)
    out["scale"] = 1.0 / np.sqrt(d)
    return out


def long_causal_inputs():
    s = WORKLOADS["long_causal"].sizes
    return causal_inputs(s["B"], s["Tq"], s["Hq"], s["d"], "bf16", s["seed"])


def layer_inputs(layer: int, T=256, H=20, d=128, seed=1004):
    """One layer's saved forward state: h (RMSNorm input), K, V caches, W, gamma.

    Layers are seeded independently with SeedSequence([seed, layer]); each layer's
    saved set only has to be internally consistent for its backward.
    """
    C = H * d
    rng = np.random.default_rng(np.random.SeedSequence([seed, layer]))
    h = normal(rng, (T, C))
    K = normal(rng, (T, H, d))
    V = normal(rng, (T, H, d))
    W = normal(rng, (C, C), std=0.02)
    gamma = uniform(rng, (C,), 0.5, 1.5)
    return dict(h=h, K=K, V=V, W=W, gamma=gamma)


def layer_upstream_grad(T=256, H=20, d=128, seed=1004):
    """The gradient arriving at the top of the layer stack, N(0, 1)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 1_000_000]))
    return normal(rng, (T, H * d))


def layernorm_inputs(rows: int, n: int, dtype: str = "f32", seed: int = 1006):
    """LayerNorm rows x and upstream gradient dy, N(0, 1) with a per-row offset and scale
    (x = 0.5 + 2 z) so the forward's centring and scaling both matter."""
    rng = np.random.default_rng(seed)
    x = normal(rng, (rows, n), std=2.0, dtype="f32") + np.float32(0.5)
    dy = normal(rng, (rows, n), dtype=dtype)
    return dict(x=_store(x.astype(np.float64), dtype), dy=dy)


def relu2_inputs(n: int, dtype: str = "f32", seed: int = 1007):
    """gate, up, dh for the ReLU^2 x Mul gate: all N(0, 1), so about half the gates are closed."""
    rng = np.random.default_rng(seed)
    return dict(gate=normal(rng, (n,), dtype=dtype), up=normal(rng, (n,), dtype=dtype), dh=normal(rng, (n,), dtype=dtype))


def ffn_inputs(T: int = 256, C: int = 2560, F: int = 6912, seed: int = 1008):
    """One FFN block's parameters and input: x, dout N(0, 1); gamma1, gamma2 U(0.5, 1.5);
    Wgu [C, 2F] and Wdown [F, C] N(0, 0.02 std). fp32."""
    rng = np.random.default_rng(seed)
    x = normal(rng, (T, C))
    gamma1 = uniform(rng, (C,), 0.5, 1.5)
    w_gu = normal(rng, (C, 2 * F), std=0.02)
    gamma2 = uniform(rng, (F,), 0.5, 1.5)
    w_down = normal(rng, (F, C), std=0.02)
    dout = normal(rng, (T, C))
    return dict(x=x, gamma1=gamma1, w_gu=w_gu, gamma2=gamma2, w_down=w_down, dout=dout)


def block_inputs(B: int = 1, T: int = 256, H: int = 20, d: int = 128, seed: int = 1009):
    """One attention block's input and weights: xin, dx2 N(0, 1); Wqkv [C, 3C] and Wo [C, C]
    N(0, 0.02 std). fp32."""
    rng = np.random.default_rng(seed)
    C = H * d
    xin = normal(rng, (B * T, C))
    w_qkv = normal(rng, (C, 3 * C), std=0.02)
    w_o = normal(rng, (C, C), std=0.02)
    dx2 = normal(rng, (B * T, C))
    return dict(xin=xin, w_qkv=w_qkv, w_o=w_o, dx2=dx2)


def rms_block_inputs(B: int = 1, T: int = 256, H: int = 20, d: int = 128, seed: int = 1010, w_std: float = 0.02):
    """One Hesper-form attention layer's input and parameters: x, dx2 N(0, 1); gamma
    U(0.5, 1.5); Wqkv [C, 3C] and Wo [C, C] N(0, w_std). fp32."""
    rng = np.random.default_rng(seed)
    C = H * d
    x = normal(rng, (B * T, C))
    gamma = uniform(rng, (C,), 0.5, 1.5)
    w_qkv = normal(rng, (C, 3 * C), std=w_std)
    w_o = normal(rng, (C, C), std=w_std)
    dx2 = normal(rng, (B * T, C))
    return dict(x=x, gamma=gamma, w_qkv=w_qkv, w_o=w_o, dx2=dx2)
