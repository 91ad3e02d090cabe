"""The host planner and the C ABI's host paths under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): the planner-parity tests (every workload's tables
bit for bit against the oracle planner, random layouts, Q groups, the hand-worked order
layouts and the rejected descriptors) run in a child process against the sanitized
build of the library, with the sanitizer runtime preloaded; any report aborts the run."""
import os
import subprocess
import sys

from block_sparse_attention_11_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sanitized_library_is_current():
    if not os.path.exists(B.SAN_OUT):
        return False
    built = os.path.getmtime(B.SAN_OUT)
    csrc = os.path.join(os.path.dirname(os.path.abspath(B.__file__)), "csrc")
    sources = [os.path.join(csrc, f) for f in os.listdir(csrc)] + [os.path.join(ROOT, "include", "kpage.h")]
    return all(os.path.getmtime(f) <= built for f in sources)


def test_planner_and_abi_host_code_clean_under_asan_and_ubsan():
    # rebuilt when a source changed since the last sanitized build (plain builds leave it)
    lib = B.SAN_OUT if _sanitized_library_is_current() else B.build_sanitized()
    env = dict(os.environ, KPAGE_LIB=lib, LD_PRELOAD=B.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the Q-group cases of the independent-partition workload repeat what the other
    # cases cover and take most of the time under the sanitizers
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_planner_parity.py", "-x", "-q", "-p",
                        "no:cacheprovider", "-k", "not (q_groups_bit_exact and 5-heads)"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
