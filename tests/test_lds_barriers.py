"""Static check of the kernels' gfx950 assembly (CPU only: hipcc cross-compiles): no
workgroup barrier is reached while an LDS write of the same wave may still be in flight.

s_barrier does not wait for a wave's outstanding LDS operations, and on gfx950 the
compiler inserts no wait before it, so every LDS write that another wave reads after a
barrier needs an explicit s_waitcnt lgkmcnt(0) first.  The scan follows each kernel's
instructions in order (branch arms included) and flags an s_barrier met after an LDS
write with no lgkmcnt(0) wait in between; only this library's kernels are checked.
"""
import os
import re
import shutil
import subprocess

import pytest

from block_sparse_attention_11_amd import build as B

CSRC = os.path.join(os.path.dirname(os.path.abspath(B.__file__)), "csrc")
SOURCES = ["fwd.hip", "bwd.hip", "select.hip", "plan_dev.hip"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def unguarded_barriers(asm: str):
    found, fn, pending = [], None, False
    for line in asm.split("\n"):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            fn, pending = m.group(1), False
            continue
        t = line.strip()
        if re.match(r"ds_(write|store)", t):
            pending = True
        elif t.startswith("s_waitcnt") and "lgkmcnt(0)" in t:
            pending = False
        elif t.startswith("s_barrier"):
            if pending and fn and fn.startswith("_ZN5kpage"):
                found.append(fn)
            pending = False
    return found


def test_scan_flags_a_barrier_after_an_unwaited_lds_write():
    asm = "_ZN5kpage1kEv:\n\tds_write_b32 v0, v1\n\ts_barrier\n\tds_write_b32 v0, v1\n" \
          "\ts_waitcnt lgkmcnt(0)\n\ts_barrier\n"
    assert unguarded_barriers(asm) == ["_ZN5kpage1kEv"]


@pytest.mark.parametrize("src", SOURCES)
def test_no_barrier_with_an_lds_write_in_flight(src, tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    out = tmp_path / (src + ".s")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-I", os.path.join(os.path.dirname(CSRC), "..", "include"),
                    "-I", CSRC, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)],
                   check=True, capture_output=True, timeout=600)
    assert unguarded_barriers(out.read_text()) == []
