"""The C-ABI layer's validation under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

fa_api.cpp (host code only) is compiled with g++ -fsanitize=address,undefined and linked with
launch stubs that answer as a launch does without a GPU (tests/host_check/launch_stubs.cpp).
tests/test_abi.py's validation cases then run against that build in a child process with the
sanitizer runtime preloaded: every case must still get its status code (a rejected argument that
reached a stub would get FA_ERR_HIP instead), with no sanitizer report.  The build uses g++ on host code alone; no GPU code is compiled with a sanitizer."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_126_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _libasan():
    p = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.timeout(600)
def test_abi_validation_under_asan_and_ubsan(tmp_path):
    if shutil.which("g++") is None or _libasan() is None:
        pytest.fail("g++ with libasan is required for the host sanitizer build")
    lib = str(tmp_path / "libfa_hostcheck.so")
    cmd = ["g++", "-std=c++17", "-shared", "-fPIC", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "fa_api.cpp"), os.path.join(ROOT, "tests", "host_check", "launch_stubs.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lamdhip64", "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, FA_ABI_TEST_LIB=lib, LD_PRELOAD=_libasan(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                        "-p", "no:cacheprovider", "-k", "validation or status or workspace_bytes"],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=500)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert r.returncode == 0, out[-3000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out
    assert " passed" in out
