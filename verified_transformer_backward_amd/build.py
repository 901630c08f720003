"""Build libvtb.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: python -m verified_transformer_backward_amd.build   (or call build()).
Every call recompiles every source; objects go to csrc/_build/, the library to
verified_transformer_backward_amd/libvtb.so. A second, separate library,
libvtb_probe.so, holds the matrix-core rate probe the benchmark reports beside the
published peaks; it is not part of the C ABI.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(CSRC, "_build")
LIB = os.path.join(HERE, "libvtb.so")
PROBE_LIB = os.path.join(HERE, "libvtb_probe.so")
PROBE_SOURCES = ["probe_peak.hip"]

SOURCES = ["api.cpp", "attn_flash_bwd.hip", "attn_bwd_mfma.hip", "attn_decode.hip", "attn_decode_fwd.hip", "elementwise.hip", "gemm_f32.hip", "ffn_norm.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libvtb)")


def _compile(src: str) -> str:
    out = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return out


def _link(objs, lib: str):
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES) + len(PROBE_SOURCES), os.cpu_count() or 4)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
