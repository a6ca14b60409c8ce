"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):

  * the oracle (oracle/ssm_oracle.c), every entry point on exact-size heap
    buffers over edge shapes (tests/sanitize/oracle_driver.c), with leak
    detection;
  * the library's C ABI, host side: the workspace-size queries over ordinary
    and extreme sizes and every entry point's argument validation on calls
    it must refuse (tests/sanitize/abi_driver.c), the library built from
    its own sources with the sanitizers on the host pass only (device code
    is compiled as usual and never launched: no GPU is needed).

A sanitizer report makes the program exit non-zero (no recovery)."""
import os
import shutil
import subprocess

import pytest

# the library's own source list, so that a new translation unit is covered too
from selective_state_space_64_amd._build import SOURCES as LIB_SOURCES

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_64_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")


def _hipcc():
    path = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return path if os.path.exists(path) else shutil.which("hipcc")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(SAN, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "ssm_oracle.c"), "-o", exe, "-lm", "-lpthread"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([exe], env=env)
    assert "oracle sanitizer run: ok" in r.stdout


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_abi_validation_under_asan_ubsan(tmp_path):
    hipcc = _hipcc()
    # sanitizers on the host pass only; the device code is built as usual
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    common = ["-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs, procs = [], []
    for src in LIB_SOURCES:
        obj = str(tmp_path / (src + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen(
            [hipcc, *common, "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", *san, "-c", os.path.join(CSRC, src), "-o", obj],
            stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    # the driver is a C caller of the ABI: compiled as C by the same compiler
    drv = str(tmp_path / "drv.o")
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = shutil.which("clang") or "gcc"
    _run([clang, "-x", "c", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(SAN, "abi_driver.c"), "-o", drv])
    for p in procs:
        out, err = p.communicate(timeout=600)
        assert p.returncode == 0, err[-4000:]
    exe = str(tmp_path / "abi_san")
    _run([hipcc, "--offload-arch=gfx950", *san, *objs, drv, "-o", exe])
    # the HIP runtime's own allocations at exit are not this library's
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([exe], env=env)
    assert "abi sanitizer run: ok" in r.stdout
