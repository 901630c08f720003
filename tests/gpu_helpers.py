"""Shared helpers of the GPU parity tests: upload exact stored values, compare with the
oracle by the max-norm relative error, print the case before each GPU step."""

import sys

import numpy as np
import pytest
import torch

import synth

# Tolerances of the parity bar: fp32 inputs 1e-4, bf16 inputs with fp32 accumulation 2e-2,
# both as max-norm relative error ||gpu - oracle||_inf / ||oracle||_inf per output tensor.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def say(*args):
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


def dev(a, dtype="f32", device="cuda:0"):
    """Upload float32 host values (bf16-exact when dtype == 'bf16') bit-exactly."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(synth.bf16_bits(a))).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref) -> float:
    """||got - ref||_inf / ||ref||_inf (the parity measure, per output tensor)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return num / den if den > 0 else num


def assert_close(name, got, ref, tol):
    e = rel_err(got, ref)
    assert np.all(np.isfinite(np.asarray(got))), f"{name}: non-finite values"
    assert e <= tol, f"{name}: max-norm relative error {e:.3e} > {tol:.1e}"
    return e
