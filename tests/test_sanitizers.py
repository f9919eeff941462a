"""The oracle and the C ABI's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

tests/sanitize/oracle_driver.c runs every oracle entry point on small
inputs and on the argument errors it must reject; tests/sanitize/
abi_driver.c drives the ABI's host validation and workspace-size queries
with calls that never reach a kernel launch.  The ABI's host translation
unit is rebuilt host-only with the sanitizers (GPU code is not
instrumented: the sanitizers apply to host code only) and linked against
the built library for the launchers it would call."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout}\n{p.stderr}"
    return p


def _check_clean(p):
    out = p.stdout + p.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
          "-fno-sanitize-recover=all", "-fopenmp", "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "dspark_oracle.c"), "-lm", "-o", exe])
    p = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "all statuses as expected" in p.stdout
    _check_clean(p)


def test_abi_host_code_under_sanitizers(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    lib_dir = os.path.join(ROOT, "rank_markov_draft_amd")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not available")
    if not os.path.exists(os.path.join(lib_dir, "libdspark_markov.so")):
        pytest.skip("libdspark_markov.so is not built")
    host_o, drv_o, exe = (str(tmp_path / n) for n in ("dspark_markov.o", "abi_driver.o", "abi_driver"))
    csrc = os.path.join(lib_dir, "csrc")
    _run([hipcc, "--offload-arch=gfx950", "--cuda-host-only", "-O1", "-g", "-std=c++17", "-ffp-contract=off",
          "-I", os.path.join(ROOT, "include"), "-Xarch_host", "-fsanitize=address", "-Xarch_host",
          "-fsanitize=undefined", "-fno-omit-frame-pointer", "-c", os.path.join(csrc, "dspark_markov.hip"),
          "-o", host_o])
    _run([clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-I",
          os.path.join(ROOT, "include"), "-c", os.path.join(SAN, "abi_driver.c"), "-o", drv_o])
    _run([clang + "++", "-fsanitize=address,undefined", drv_o, host_o, "-L" + lib_dir, "-ldspark_markov",
          "-Wl,-rpath," + lib_dir, "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    p = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "all statuses as expected" in p.stdout
    _check_clean(p)
