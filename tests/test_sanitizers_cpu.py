"""Host sanitizers (no GPU): the C ABI's argument checks, planning queries and
entry points, and the FP64 oracle, built with AddressSanitizer and
UndefinedBehaviorSanitizer, run the CPU test files in a child process with
the sanitizer runtime preloaded.  Any report (an out-of-bounds access, a
use after free, signed overflow, a misaligned or null dereference, a shift
out of range) fails the child and this test.  The habit of running a
memory checker over every version is that of "现代 CUDA 工具箱实战：从朴素代码到
硬件极限的优化之路", section 调试技巧.

Every call the child makes is rejected before a device call or finds no
device (the C-ABI tests use fake addresses and are written so that none of
them reaches a launch), so the instrumented host code is exercised while no
kernel runs.  The sanitized builds are made on first use (about a minute for
the library) and reused after that.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

CPU_FILES = ["test_boundary_cpu.py", "test_splitk_boundary_cpu.py", "test_streamk_boundary_cpu.py",
             "test_lowp_boundary_cpu.py", "test_transpose_boundary_cpu.py", "test_device_status_cpu.py",
             "test_oracle_pins.py", "test_oracle_lowp_pins.py", "test_oracle_transpose_pins.py"]


def _built(path, sources):
    return os.path.exists(path) and all(os.path.getmtime(path) >= os.path.getmtime(s) for s in sources)


@pytest.fixture(scope="module")
def sanitized():
    from fp32_gemm_08_amd import build as hipbuild
    import oracle

    try:
        runtime = hipbuild.sanitizer_runtime()
    except (RuntimeError, FileNotFoundError) as e:
        pytest.skip(f"no clang sanitizer runtime: {e}")
    lib = hipbuild.variant_path("sanitize")
    srcs = [os.path.join(hipbuild.CSRC, s) for s in hipbuild.SOURCES] + \
        [os.path.join(hipbuild.CSRC, h) for h in os.listdir(hipbuild.CSRC) if h.endswith(".h")] + \
        [os.path.join(ROOT, "include", "sgemm_f32.h")]
    if not _built(lib, srcs):
        hipbuild.build(variant="sanitize")
    if not _built(oracle.ORACLE_SANITIZE_SO, [oracle.ORACLE_SRC]):
        oracle.build_sanitized()
    return runtime, lib, oracle.ORACLE_SANITIZE_SO


def test_cpu_suites_under_asan_and_ubsan(sanitized):
    runtime, lib, oracle_so = sanitized
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtime,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1:detect_stack_use_after_return=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "SGEMM_F32_LIBRARY": lib,
        "SGEMM_ORACLE_LIBRARY": oracle_so,
        "HIP_VISIBLE_DEVICES": "-1",
    })
    files = [os.path.join(ROOT, "tests", f) for f in CPU_FILES]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"] + files,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout.splitlines()[-1], r.stdout[-2000:]


def test_the_child_really_runs_sanitized(sanitized):
    """The preload and the library overrides take effect: the child loads the
    sanitized builds, and a planted out-of-bounds read (the oracle told that a
    4 x 4 A has 8 columns) is reported by AddressSanitizer."""
    runtime, lib, oracle_so = sanitized
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0", SGEMM_F32_LIBRARY=lib,
               SGEMM_ORACLE_LIBRARY=oracle_so, HIP_VISIBLE_DEVICES="-1")
    child = (
        "import sys, ctypes; sys.path.insert(0, sys.argv[1])\n"
        "import numpy as np\n"
        "import fp32_gemm_08_amd as lib, oracle\n"
        "assert lib.LIB_PATH == sys.argv[2] and oracle.ORACLE_SO == sys.argv[3]\n"
        "assert 'ASan' in lib.sgemm_f32_version()\n"
        "o = oracle.load_library(oracle.ORACLE_SO)\n"
        "print('loaded', flush=True)\n"
        "A = np.ones((4, 4), np.float32); B = np.ones((8, 4), np.float32)\n"
        "rows = np.arange(4, dtype=np.int64); D = np.zeros((4, 4)); S = np.zeros((4, 4))\n"
        "p = lambda x: x.ctypes.data_as(ctypes.c_void_p)\n"
        "o.oracle_gemm_rows(4, 4, 8, 1.0, p(A), 8, p(B), 4, 0, 0.0, None, 4, p(rows), 4, p(D), p(S), 1)\n"
        "print('not reported', flush=True)\n"
    )
    r = subprocess.run([sys.executable, "-c", child, ROOT, lib, oracle_so], env=env, capture_output=True, text=True,
                       timeout=120)
    assert "loaded" in r.stdout, r.stderr[-2000:]
    assert "not reported" not in r.stdout
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr and "oracle_gemm" in r.stderr, r.stderr[-3000:]
