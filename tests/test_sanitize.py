"""The C oracle and the C ABI's host-side checks under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).  Each builds its own instrumented copy
in a temporary directory and runs a driver (tests/sanitize/) that calls every
entry point: the oracle on small inputs with format edge cases, the ABI with
out-of-contract arguments that it must refuse before any HIP call."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{cmd[0]} failed ({r.returncode}):\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Wno-unknown-pragmas",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "k3oracle.c"), os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    r = _run([exe], env=ENV)
    assert "oracle driver ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs hipcc")
def test_abi_checks_under_sanitizers(tmp_path):
    from mxfp4_routed_expert_softmax_amd import build as b
    lib = str(tmp_path / "libk3moe_san.so")
    # the library's own flags, host code instrumented (device code untouched);
    # -z defs would reject the sanitizer runtime's symbols, which the driver provides
    flags = [f for f in b.FLAGS if f not in ("-O3", "-Wl,-z,defs")]
    host = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]
    srcs = [os.path.join(b.CSRC, s) for s in b.SOURCES]
    _run([HIPCC, *flags, "-O1", "-g", *host, "-I", os.path.join(ROOT, "include"), "-I", b.CSRC, *srcs, "-o", lib])
    exe = str(tmp_path / "abi_driver")
    _run([CLANG, "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
          os.path.join(HERE, "abi_driver.c"), lib, "-Wl,-rpath," + str(tmp_path), "-o", exe])
    r = _run([exe], env=ENV)
    assert "abi driver ok" in r.stdout
