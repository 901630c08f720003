"""Every barrier in the library's kernels follows completed LDS stores (see isa_barriers)."""

import concurrent.futures
import os
import shutil
import subprocess
import tempfile

import pytest

from verified_transformer_backward_amd import build as B
from isa_barriers import kernel_bodies, unsafe_barriers

HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)
HIP_SOURCES = [s for s in B.SOURCES if s.endswith(".hip")]


def _asm(src: str, tmp: str) -> str:
    out = os.path.join(tmp, src + ".s")
    flags = [f for f in B.FLAGS if f != "-fPIC"]
    subprocess.run([HIPCC, *flags, "-x", "hip", "-S", "--cuda-device-only", os.path.join(B.CSRC, src), "-o", out],
                   check=True, capture_output=True)
    return open(out).read()


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
def test_no_barrier_before_lds_stores_complete():
    with tempfile.TemporaryDirectory() as tmp:
        with concurrent.futures.ThreadPoolExecutor(min(len(HIP_SOURCES), os.cpu_count() or 4)) as ex:
            listings = dict(zip(HIP_SOURCES, ex.map(lambda s: _asm(s, tmp), HIP_SOURCES)))
    bad, n = [], 0
    for src, asm in listings.items():
        for name, lines in kernel_bodies(asm):
            n += 1
            lab = unsafe_barriers(lines)
            if lab:
                bad.append(f"{src}: {name} at {lab}")
    assert n > 20, "expected the library's kernels in the listings"
    assert not bad, "barrier reachable with pending LDS stores:\n" + "\n".join(bad)


def test_checker_flags_a_missing_wait():
    """The checker itself: a loop whose back edge reaches the barrier right after a store."""
    lines = """
.LBB0_1:
	s_barrier
	ds_read_b128 v[0:3], v4
	s_waitcnt lgkmcnt(0)
	ds_write_b128 v5, v[0:3]
	s_cbranch_scc1 .LBB0_1
	s_endpgm
""".split("\n")
    assert unsafe_barriers(lines) == [".LBB0_1"]
    fixed = [ln.replace("s_cbranch_scc1", "s_waitcnt lgkmcnt(0)\n\ts_cbranch_scc1") for ln in lines]
    fixed = "\n".join(fixed).split("\n")
    assert unsafe_barriers(fixed) == []
