"""Numerical-gradient verification, as the "Hesper.Training.VerifiedBackward" page's section
"Numerical Gradient Verification" describes it, plus the wrong-backward set of the Hesper
commit log. Test infrastructure only.

Readings of the unrendered bodies:
  * numericalGrad(f, x, eps=1e-4): central differences (f(x + eps e_i) - f(x - eps e_i)) / (2 eps)
    of a scalar f, one coordinate at a time.
  * checkGradient(analytical, numerical, tol=1e-3): pass iff
    max_i |a_i - n_i| <= tol * max(1, max_i |n_i|).
  * A vector-valued op F is checked through the scalar L(x) = <dy, F(x)>, whose gradient
    is exactly the VJP F'(x)^T dy that the backward spec returns.
"""

from __future__ import annotations

from typing import Callable

import numpy as np

from . import specs
from .attention import attention_backward, attention_forward
from .layer import rope_backward_rows, rope_forward_rows


def numerical_grad(f: Callable[[np.ndarray], float], x, eps: float = 1e-4) -> np.ndarray:
    x = np.array(x, dtype=np.float64)
    g = np.zeros_like(x)
    flat, gflat = x.reshape(-1), g.reshape(-1)
    for i in range(flat.size):
        keep = flat[i]
        flat[i] = keep + eps
        fp = f(x)
        flat[i] = keep - eps
        fm = f(x)
        flat[i] = keep
        gflat[i] = (fp - fm) / (2.0 * eps)
    return g


def gradient_error(analytical, numerical) -> float:
    a, n = np.asarray(analytical, np.float64), np.asarray(numerical, np.float64)
    return float(np.max(np.abs(a - n))) if a.size else 0.0


def check_gradient(analytical, numerical, tol: float = 1e-3) -> bool:
    n = np.asarray(numerical, np.float64)
    scale = max(1.0, float(np.max(np.abs(n))) if n.size else 0.0)
    return gradient_error(analytical, numerical) <= tol * scale


def vjp_loss(forward: Callable[[np.ndarray], np.ndarray], dy) -> Callable[[np.ndarray], float]:
    dy = np.asarray(dy, np.float64)
    return lambda x: float(np.sum(dy * forward(x)))


def softmax_numerical_check(x, target_idx: int, eps: float = 1e-5) -> bool:
    """softmaxNumericalCheck: the gradient of s_target with respect to x, computed by
    softmaxBackward with a one-hot dy, agrees with central differences."""
    x = np.asarray(x, np.float64)
    dy = np.zeros_like(x)
    dy[target_idx] = 1.0
    analytical = specs.softmax_backward(x, dy)
    numerical = numerical_grad(lambda z: float(specs.softmax_forward(z)[target_idx]), x, eps)
    return check_gradient(analytical, numerical)


# ----------------------------------------------------------------------------- wrong backwards

def wrong_backwards():
    """The commit log's wrong-backward set: each maps (correct_vjp, dy) -> a wrong result.
    'wrong_rope_sign' only applies to RoPE: it rotates by +theta instead of -theta."""
    return {
        "zero": lambda vjp, dy: np.zeros_like(vjp),
        "identity": lambda vjp, dy: np.asarray(dy, np.float64).reshape(vjp.shape) if np.size(dy) == np.size(vjp) else np.ones_like(vjp),
        "negated": lambda vjp, dy: -vjp,
    }


def rope_backward_wrong_sign(dy, pos, base=10000.0, layout=0):
    """R(+theta) applied to dy: the forward rotation used where the inverse belongs."""
    return rope_forward_rows(dy, pos, base, layout)


# ----------------------------------------------------------------------------- verify*

def verify_softmax_backward(n: int = 5, seed: int = 0, backward=None) -> bool:
    rng = np.random.default_rng(seed)
    x, dy = rng.standard_normal(n), rng.standard_normal(n)
    bwd = backward or specs.softmax_backward
    num = numerical_grad(vjp_loss(specs.softmax_forward, dy), x)
    return check_gradient(bwd(x, dy), num)


def verify_rope_backward(T: int = 3, H: int = 1, d: int = 8, pos0: int = 5, seed: int = 0, backward=None) -> bool:
    rng = np.random.default_rng(seed)
    x, dy = rng.standard_normal((T, H, d)), rng.standard_normal((T, H, d))
    pos = pos0 + np.arange(T)
    bwd = backward or rope_backward_rows
    num = numerical_grad(vjp_loss(lambda z: rope_forward_rows(z, pos), dy), x)
    return check_gradient(bwd(dy, pos), num)


def verify_rmsnorm_backward(n: int = 8, seed: int = 0, eps: float = 1e-6, backward=None) -> bool:
    rng = np.random.default_rng(seed)
    x, dy = rng.standard_normal(n), rng.standard_normal(n)
    gamma = rng.uniform(0.5, 1.5, n)
    bwd = backward or (lambda x_, g_, dy_: specs.rmsnorm_backward(x_, g_, dy_, eps))
    num = numerical_grad(vjp_loss(lambda z: specs.rmsnorm_forward(z, gamma, eps), dy), x)
    return check_gradient(bwd(x, gamma, dy), num)


def verify_attention_backward(B=1, Tq=3, Tk=4, Hq=2, Hkv=1, d=4, causal=True, seed=0) -> dict:
    """Central differences of L = <dO, Attention(q, k, v)> against dq, dk, dv."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Tq, Hq, d))
    k = rng.standard_normal((B, Tk, Hkv, d))
    v = rng.standard_normal((B, Tk, Hkv, d))
    do = rng.standard_normal((B, Tq, Hq, d))
    scale = 1.0 / np.sqrt(d)
    dq, dk, dv = attention_backward(q, k, v, do, scale, causal)
    fq = lambda z: float(np.sum(do * attention_forward(z, k, v, scale, causal)[0]))
    fk = lambda z: float(np.sum(do * attention_forward(q, z, v, scale, causal)[0]))
    fv = lambda z: float(np.sum(do * attention_forward(q, k, z, scale, causal)[0]))
    return dict(dq=check_gradient(dq, numerical_grad(fq, q)),
                dk=check_gradient(dk, numerical_grad(fk, k)),
                dv=check_gradient(dv, numerical_grad(fv, v)))


def run_all_checks(verbose: bool = True) -> bool:
    """runAllChecks: every verify* plus the Tier-1 identities of the page's
    "Verification Strategy" (RoPE roundtrip, softmax gradient sums to zero)."""
    results = {
        "softmax_fd": verify_softmax_backward(),
        "softmax_numerical_check": softmax_numerical_check([0.3, -1.2, 2.0, 0.1], 2),
        "softmax_sums_to_zero": abs(specs.softmax_backward_sums_to_zero([1.0, 2.0, 3.0], [0.5, -1.0, 2.0])) < 1e-12,
        "rope_fd": verify_rope_backward(),
        "rope_roundtrip": specs.rope_roundtrip_check(0.7, -1.3, 5.0),
        "rmsnorm_fd": verify_rmsnorm_backward(),
        **{f"attention_fd_{k}": v for k, v in verify_attention_backward().items()},
    }
    if verbose:
        for name, ok in results.items():
            print(f"{name:32s} {'PASS' if ok else 'FAIL'}")
    return all(results.values())
