"""The C ABI's host code and the oracle built with the address and undefined-behaviour sanitizers and run
on the CPU (no GPU): tests/sanitize/abi_driver.cpp drives abi.cpp's validation, planning and dispatch with
stub launchers; tests/sanitize/oracle_driver.c runs every oracle entry point on small and edge-case inputs.
A sanitizer report, or a status other than the expected one, fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "selective_state_space_82_amd", "csrc")
ROCM = "/opt/rocm"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "oracle"), os.path.join(HERE, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "ssm_oracle.c"), "-lm", "-o", exe])
    r = _run([exe], env=ENV)
    assert "every entry point ran clean" in r.stdout
    assert "runtime error" not in r.stderr


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "bin", "hipcc")), reason="needs the ROCm toolchain")
def test_abi_host_code_under_sanitizers(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang++")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src in (os.path.join(CSRC, "abi.cpp"), os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "abi_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([hipcc, "-O1", "-g", "-std=c++17", "-fPIC"] + san + inc + ["-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "abi_driver")
    # host-only link with the sanitizer runtimes (no device code in these objects)
    _run([clang, "-fsanitize=address,undefined"] + objs + ["-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                                                            "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    r = _run([exe], env=ENV)
    assert "all host paths behaved" in r.stdout, r.stdout
    assert "runtime error" not in r.stderr
