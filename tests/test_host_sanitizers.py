"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the C
ABI's validation, launch planning and workspace layout (favor_api.cpp and
favor_plan.cpp with the kernel launcher replaced by a checking stub), the
host projection generator (orf_omega.cpp) and the plain-C oracle
(favor_oracle.c) are compiled with g++/gcc and both sanitizers and driven over
wide grids of shapes, plans and invalid arguments (tests/sanitize/)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(SAN, "_build")
CSRC = os.path.join(ROOT, "positive_random_feature_amd", "csrc")
FLAGS = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, **kw)


@pytest.fixture(scope="module")
def outdir():
    if shutil.which("g++") is None or shutil.which("gcc") is None:
        pytest.skip("no host compiler")
    os.makedirs(OUT, exist_ok=True)
    return OUT


def test_abi_host_code_sanitized(outdir):
    exe = os.path.join(outdir, "abi_driver")
    cmd = ["g++", "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(SAN, "abi_driver.cpp"), os.path.join(SAN, "stub_launch.cpp"),
           os.path.join(CSRC, "favor_api.cpp"), os.path.join(CSRC, "favor_plan.cpp"),
           os.path.join(CSRC, "orf_omega.cpp"), "-o", exe]
    b = _run(cmd)
    assert b.returncode == 0, b.stderr[-4000:]
    r = _run([exe], env=ENV, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "0 failures" in r.stdout


def test_oracle_sanitized(outdir):
    exe = os.path.join(outdir, "oracle_driver")
    cmd = ["gcc", "-std=c11", *FLAGS, os.path.join(SAN, "oracle_driver.c"),
           os.path.join(ROOT, "oracle", "favor_oracle.c"), "-lm", "-o", exe]
    b = _run(cmd)
    assert b.returncode == 0, b.stderr[-4000:]
    r = _run([exe], env=ENV, timeout=300)
    assert r.returncode == 0, (r.stdout, r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "oracle_driver: ok" in r.stdout
