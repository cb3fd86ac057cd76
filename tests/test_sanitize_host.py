"""Host builds of the C ABI's validation layer and of the C oracle under
AddressSanitizer and UndefinedBehaviorSanitizer.

The ABI source (api.hip) holds no device code: it validates arguments and
calls the launchers.  It is compiled here by g++ as C++ (a copy named .cpp),
linked against host-only stand-ins of the launchers (tests/sanitize/stubs.cpp)
and driven with valid and invalid arguments (tests/sanitize/abi_driver.cpp):
every invalid call must return its documented status, every valid one must
reach the stand-in launcher, and no check may read an operand, overflow a
signed integer or wrap a size.  The oracle is built with gcc and driven over
every function with exact-extent buffers (tests/sanitize/oracle_driver.c).
No GPU and no HIP runtime is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "invariant_gemm_amd", "csrc")
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not found")


def _build(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower() and "cannot find" in r.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stderr[-4000:]


def _run(exe, cwd):
    r = subprocess.run([exe], cwd=cwd, capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert "all checks passed" in r.stdout


def test_abi_validation_under_sanitizers(tmp_path):
    _need("g++")
    src = tmp_path / "api.cpp"
    shutil.copyfile(os.path.join(CSRC, "api.hip"), src)
    exe = str(tmp_path / "abi")
    _build(["g++", "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
            f"-I{CSRC}", f"-I{os.path.join(ROOT, 'include')}", str(src),
            os.path.join(SAN, "stubs.cpp"), os.path.join(SAN, "abi_driver.cpp"), "-o", exe],
           tmp_path)
    _run(exe, tmp_path)


def test_oracle_under_sanitizers(tmp_path):
    _need("gcc")
    exe = str(tmp_path / "ora")
    _build(["gcc", "-std=c11", *FLAGS, "-fopenmp", os.path.join(ROOT, "oracle", "oracle.c"),
            os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe], tmp_path)
    _run(exe, tmp_path)
