"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Builds the library's HIP sources together with tests/abi_host_check.hip, with both sanitizers
on the host code only (each -fsanitize behind -Xarch_host; the GPU code is built as usual), and
runs the checks: argument validation of every entry point, workspace sizes over shapes up to
the int32 limits, the refusals made before any launch, status strings and the host analytics.
Nothing in the program touches a GPU.  Leak detection is off: the HIP runtime's own start-up
allocations are not this code's.
"""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_sampling_verification_amd", "csrc")
SOURCES = ["sv_kernels.hip", "sv_rest.hip", "sv_rng.hip", "sv_abi.hip"]


def _hipcc():
    path = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return path if os.path.exists(path) else None


@pytest.mark.timeout(1200)
def test_abi_host_code_under_sanitizers(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "abi_host_check")
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES],
           os.path.join(ROOT, "tests", "abi_host_check.hip"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=1100)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    print(run.stdout[-2000:])
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-3000:]
    assert " 0 failures" in run.stdout
