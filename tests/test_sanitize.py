"""The CPU suite under address and undefined-behaviour sanitizers (CPU only).

Two sanitized builds, both with ROCm's clang so that one sanitizer runtime
serves the process:
  * the oracle (oracle/ep_oracle.c) with -fsanitize=address,undefined;
  * the HIP library with the sanitizers on its host code only (each
    -fsanitize= behind -Xarch_host; the gfx950 device code is built as usual
    and never runs here).
The rest of the CPU suite then runs in a child process with the sanitizer
runtime preloaded and EP_HIP_LIB / EP_ORACLE_LIB pointing at those builds:
every host-side path -- argument validation, workspace and LDS sizing at the
ABI limits, accounting, the plain-C oracle with its threaded mode, the
worked-example pin -- runs instrumented, and any report fails the test.  A
second child checks the sanitizer is live: it makes the oracle copy a row to
a slot past its buffer (a mistake planted on the CPU) and must be stopped
with a heap-buffer-overflow report.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
_RT = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
ASAN_RT = _RT[-1] if _RT else None

pytestmark = pytest.mark.skipif(not (ASAN_RT and os.path.exists(CLANG) and os.path.exists(HIPCC)),
                                reason="ROCm clang / hipcc or clang's ASan runtime not installed")

SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    sys.path.insert(0, ROOT)
    from combine_dispatch_layout_02_amd import build as hip_build

    out = tmp_path_factory.mktemp("sanitized")
    oracle_lib = str(out / "libep_oracle.so")
    subprocess.run([CLANG, "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", *SANITIZE,
                    "-shared-libsan", "-fPIC", "-shared", os.path.join(ROOT, "oracle", "ep_oracle.c"),
                    "-o", oracle_lib, "-lm"], check=True)
    hip_lib = str(out / "libep_hip.so")
    host_only = []
    for flag in SANITIZE:
        host_only += ["-Xarch_host", flag]
    subprocess.run([HIPCC, *hip_build.HIPCC_FLAGS, *host_only, "-shared-libsan",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(hip_build.PKG, "csrc"),
                    "-o", hip_lib, *hip_build.sources()], check=True, stderr=subprocess.DEVNULL)
    env = dict(os.environ, LD_PRELOAD=ASAN_RT, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", EP_HIP_LIB=hip_lib,
               EP_ORACLE_LIB=oracle_lib)
    return env, hip_lib, oracle_lib


def test_cpu_suite_runs_clean_under_sanitizers(sanitized):
    env, hip_lib, oracle_lib = sanitized
    # the sanitized builds are the ones that load
    probe = ("import sys; sys.path.insert(0, %r)\n"
             "from combine_dispatch_layout_02_amd import ep\nimport oracle\n"
             "ep.load(); oracle._load()\n"
             "maps = open('/proc/self/maps').read()\n"
             "assert %r in maps and %r in maps, 'sanitized builds not loaded'\n" % (ROOT, hip_lib, oracle_lib))
    subprocess.run([sys.executable, "-c", probe], env=env, check=True, timeout=300)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "-k", "not sanitize", os.path.join(ROOT, "tests")],
                       env=env, capture_output=True, text=True, timeout=1500)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stdout + r.stderr, report
    assert "runtime error:" not in r.stdout + r.stderr, report


def test_sanitizer_is_live(sanitized):
    env, _, _ = sanitized
    planted = ("import sys; sys.path.insert(0, %r)\n"
               "import numpy as np, oracle\n"
               "lib = oracle._load()\n"
               "src = np.zeros((4, 64), np.uint8)\n"
               "slots = np.array([[0], [1], [2], [5]], np.int32)   # slot 5 of a 4-row buffer\n"
               "recv = np.zeros((4, 64), np.uint8)\n"
               "lib.oracle_dispatch_rows(4, 1, 64, oracle._p(src), oracle._p(slots), oracle._p(recv))\n" % ROOT)
    r = subprocess.run([sys.executable, "-c", planted], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
