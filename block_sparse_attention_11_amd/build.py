"""Build libkpage.so in-tree with hipcc for gfx950.

    python -m block_sparse_attention_11_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["csrc/plan.cpp", "csrc/api.hip", "csrc/plan_dev.hip", "csrc/fwd.hip", "csrc/bwd.hip", "csrc/select.hip"]
OUT = os.path.join(HERE, "libkpage.so")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from forming packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]
# Per-source extras (none at present).
EXTRA: dict = {}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


# Host code of the planner and the C ABI, built again with AddressSanitizer and
# UndefinedBehaviorSanitizer for the CPU tests (GPU code is never sanitized: each
# sanitizer option applies to the host pass only).
SANITIZED = ["csrc/plan.cpp", "csrc/api.hip"]
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xarch_host", "-shared-libasan"]
SAN_OUT = os.path.join(HERE, "_build", "libkpage_san.so")


def asan_runtime() -> str:
    """The compiler's shared AddressSanitizer runtime (preloaded by the sanitized test run)."""
    import glob
    rocm = os.path.dirname(os.path.dirname(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")))
    found = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under " + rocm)
    return found[-1]


def build_sanitized(verbose: bool = False) -> str:
    """libkpage_san.so: the planner and C ABI host code with ASan + UBSan, the kernels'
    objects of the regular build (built first if missing)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(HERE, "csrc")]
    objdir = os.path.join(HERE, "_build")
    plain = [os.path.join(objdir, os.path.basename(s) + ".o") for s in SOURCES if s not in SANITIZED]
    if not all(os.path.exists(o) for o in plain):
        build(verbose)
    sandir = os.path.join(objdir, "san")
    os.makedirs(sandir, exist_ok=True)
    objs = []
    for src in SANITIZED:
        obj = os.path.join(sandir, os.path.basename(src) + ".o")
        flags = [f if f != "-O3" else "-O1" for f in FLAGS] + ["-g"]
        _run([hipcc, *flags, *SAN_FLAGS, *inc, "-c", os.path.join(HERE, src), "-o", obj], verbose)
        objs.append(obj)
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN_FLAGS, *objs, *plain, "-o", SAN_OUT + ".tmp"],
         verbose)
    os.replace(SAN_OUT + ".tmp", SAN_OUT)
    return SAN_OUT


def build(verbose: bool = False) -> str:
    """Compile every source to an object (per-source flags), then link the library."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(HERE, "csrc")]
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(src) + ".o") for src in SOURCES]
    # one hipcc per source, in parallel
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as pool:
        futures = [pool.submit(_run, [hipcc, *FLAGS, *EXTRA.get(src, []), *inc, "-c", os.path.join(HERE, src), "-o", obj],
                               verbose) for src, obj in zip(SOURCES, objs)]
        for f in futures:
            f.result()
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", OUT + ".tmp"], verbose)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if "--sanitized" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
