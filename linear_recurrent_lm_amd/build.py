"""Build libwkv7.so (gfx950) in-tree with hipcc.

    python -m linear_recurrent_lm_amd.build [--resource-usage]
    python -m linear_recurrent_lm_amd.build --asan   # host code under AddressSanitizer

Every .hip file under csrc/ is compiled for gfx950 only and linked into
linear_recurrent_lm_amd/libwkv7.so; the issue-pipe probe under csrc/probe/
goes into its own libwkv7_probe.so. Packed-FP32 instruction selection is
disabled for all device code (-target-feature -packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(os.path.dirname(HERE), "_build", "obj")
LIB = os.path.join(HERE, "libwkv7.so")
PROBE_SRC = os.path.join(CSRC, "probe", "pipe_probe.hip")
PROBE_LIB = os.path.join(HERE, "libwkv7_probe.so")
ASAN_DIR = os.path.join(os.path.dirname(HERE), "_build", "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libwkv7.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src, extra):
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj, res.stderr


def build(resource_usage: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJ, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=jobs or min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), srcs))
    if resource_usage:
        for _, log in results:
            if log.strip():
                sys.stderr.write(log)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[o for o, _ in results],
           "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


def asan_runtime() -> str:
    """The compiler's AddressSanitizer runtime, which a non-instrumented
    Python must preload to load the sanitized library."""
    found = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib",
                                          "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise RuntimeError("no libclang_rt.asan-x86_64.so next to hipcc")
    return found[-1]


def build_asan() -> str:
    """Every source again with its host code under AddressSanitizer (the
    device code is built as usual, unsanitized): the argument, size and
    overlap checks run instrumented. Written to _build/asan/libwkv7.so; load
    it with WKV7_LIBRARY set to that path and the runtime from
    asan_runtime() preloaded."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    host = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]
    sanitize = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()

    def one(src):
        obj = os.path.join(ASAN_DIR, os.path.basename(src) + ".o")
        res = subprocess.run([HIPCC, *host, *sanitize, "-c", src, "-o", obj],
                             capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc (asan) failed for {src}:\n{res.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(one, sources()))
    res = subprocess.run([HIPCC, "-shared", "-fPIC", *sanitize, *objs, "-o", ASAN_LIB],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link (asan) failed:\n{res.stderr}")
    return ASAN_LIB


def build_probe() -> str:
    """The issue-pipe probe (csrc/probe/), a library of its own that only the
    measurement script loads."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", PROBE_SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PROBE_SRC}:\n{res.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    if "--asan" in sys.argv:
        print(build_asan())
    else:
        print(build(resource_usage="--resource-usage" in sys.argv))
        print(build_probe())
