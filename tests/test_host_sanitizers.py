"""Host code under AddressSanitizer + UndefinedBehaviorSanitizer (and the
threaded oracle under ThreadSanitizer): the fp64 oracles (forward and
gradients) with their thread pools,
and the C ABI's argument validation in kda_api.cpp with the kernel launchers
replaced by stubs (tests/sanitize/launch_stubs.cpp).  Each build runs a small
driver that checks its own results; any sanitizer report fails the run.
Device code is not involved: the drivers are built with gcc / g++ only."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ASAN_UBSAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer"]


def _build_and_run(cmd, exe, env_extra=None):
    res = subprocess.run(cmd + ["-o", exe], capture_output=True, text=True)
    assert res.returncode == 0, "build failed:\n" + " ".join(cmd) + "\n" + res.stderr[-3000:]
    env = dict(os.environ)
    env.update(env_extra or {})
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, "driver failed (%d):\n%s%s" % (run.returncode, run.stdout[-2000:],
                                                               run.stderr[-4000:])
    assert "passed" in run.stdout
    return run.stdout


@pytest.fixture(scope="module")
def tmp():
    d = tempfile.mkdtemp(prefix="kda_san_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_asan_ubsan(tmp):
    _build_and_run(["gcc", "-std=c99", "-D_POSIX_C_SOURCE=200809L"] + ASAN_UBSAN +
                   [os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "kda_oracle.c"),
                    os.path.join(ROOT, "oracle", "kda_oracle_bwd.c"),
                    "-lm", "-lpthread"], os.path.join(tmp, "oracle_asan"),
                   {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0"})


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_tsan(tmp):
    _build_and_run(["gcc", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-O1", "-g",
                    "-fsanitize=thread", os.path.join(SAN, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "kda_oracle.c"),
                    os.path.join(ROOT, "oracle", "kda_oracle_bwd.c"), "-lm", "-lpthread"],
                   os.path.join(tmp, "oracle_tsan"), {"TSAN_OPTIONS": "halt_on_error=1"})


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not available")
def test_abi_validation_asan_ubsan(tmp):
    _build_and_run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I" + os.path.join(ROOT, "include"), "-I" + SAN] + ASAN_UBSAN +
                   [os.path.join(SAN, "api_driver.cpp"), os.path.join(SAN, "launch_stubs.cpp"),
                    os.path.join(ROOT, "kimi_delta_attention_02_amd", "csrc", "kda_api.cpp")],
                   os.path.join(tmp, "api_asan"), {"ASAN_OPTIONS": "detect_leaks=1"})


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_sanitizer_is_live(tmp):
    """The same flags do catch a one-past-the-end heap read, so a clean run
    above means something."""
    src = os.path.join(tmp, "canary.c")
    with open(src, "w") as f:
        f.write("#include <stdlib.h>\nint main(void) { int* a = malloc(8 * sizeof(int));\n"
                "  volatile int i = 8; int x = a[i]; free(a); return x & 0; }\n")
    exe = os.path.join(tmp, "canary")
    res = subprocess.run(["gcc"] + ASAN_UBSAN + [src, "-o", exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    # AddressSanitizer's heap-buffer-overflow, or UBSan's object-size check first
    assert run.returncode != 0
    assert "heap-buffer-overflow" in run.stderr or "insufficient space" in run.stderr
