"""The host code of the library under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

A second build of the same sources instruments the host half only (each -fsanitize flag
behind -Xarch_host; the gfx950 kernels are built as usual), and the host-validation suites
(test_abi_cpu, test_linear_abi_cpu, test_grpo_abi_cpu) run against it in a child process with
the ASan runtime preloaded: every argument check, overflow guard and error path of the C
entry points executes instrumented, and any report fails the test.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from deterministic_selected_token_amd import build  # noqa: E402

SUITES = ["tests/test_abi_cpu.py", "tests/test_linear_abi_cpu.py", "tests/test_grpo_abi_cpu.py"]


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.timeout(900)
def test_host_code_under_asan_and_ubsan():
    rt = asan_runtime()
    if rt is None:
        pytest.skip("no clang ASan runtime in this image")
    tmp = tempfile.mkdtemp(prefix="san_")
    lib = os.path.join(tmp, "liblogp_mi355x_san.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-shared-libsan", "-g", "-O1"]
    cmd = [a for a in build.command(lib, san) if a != "-O3"]
    subprocess.run(cmd, check=True, capture_output=True)
    logs = os.path.join(tmp, "report")
    env = dict(os.environ, DST_AMD_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS=f"detect_leaks=0:log_path={logs}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={logs}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *SUITES], cwd=ROOT, env=env, capture_output=True,
                       text=True)
    reports = glob.glob(logs + "*")
    text = "".join(open(f).read() for f in reports)
    assert r.returncode == 0 and not reports, (r.stdout[-2000:], text[:4000])
