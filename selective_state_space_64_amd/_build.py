"""Build step: compiles the HIP sources in csrc/ for gfx950 into libssm.so
beside this file (hipcc, one object per source, compiled in parallel)."""
import concurrent.futures
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libssm.so")
PEAKS_LIB = os.path.join(HERE, "libssm_peaks.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["ssm_api.hip", "scan_fwd.hip", "scan_bld.hip", "state_update.hip", "conv1d.hip",
           "scan_bwd.hip", "transpose.hip"]
ARCH = "gfx950"
# Packed fp32 VALU ops are kept out of the generated code on purpose.
HIPFLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument"]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or path)


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPFLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    return obj


def _link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, out)


def build(verbose=False):
    """libssm.so (the library) and libssm_peaks.so (the issue-rate probes
    the benchmark reports beside the nominal peaks)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(len(SOURCES) + 1) as ex:
        objs = list(ex.map(_compile, SOURCES + ["peaks.hip"]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], PEAKS_LIB)
    if verbose:
        print("built", LIB, PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
