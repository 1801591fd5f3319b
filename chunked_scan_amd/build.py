"""Build liblachunk.so in-tree from csrc/*.hip with hipcc for gfx950.

Every HIP source is compiled to an object in parallel, then linked into one shared library next
to this file.  Packed-fp32 instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(HERE, "liblachunk.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if ln.strip() and "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, "\n".join(msgs)))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


SAN_DIR = os.path.join(ROOT, "_build", "san")
SAN_LIB = os.path.join(SAN_DIR, "liblachunk.so")
# clang's shared AddressSanitizer runtime (it carries UndefinedBehaviorSanitizer too); a process
# that loads SAN_LIB needs it preloaded: LD_PRELOAD=<asan_runtime()>
def asan_runtime() -> str:
    out = subprocess.run([HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang's AddressSanitizer runtime was not found")
    return path


def build_sanitized(verbose: bool = True) -> str:
    """The library with its host code built with AddressSanitizer and UndefinedBehaviorSanitizer
    (device code as in build(), uninstrumented) into _build/san/liblachunk.so: the argument
    validation, the planning arithmetic and the error paths of every entry point run under the
    sanitizers, also on a machine without a GPU.  Run a program against it with LACHUNK_LIB=<path>, LD_PRELOAD=<asan_runtime()>
    and ASAN_OPTIONS=detect_leaks=0 (the Python interpreter itself is not instrumented)."""
    os.makedirs(SAN_DIR, exist_ok=True)
    flags = ["-O3", "-std=c++17", "-fPIC", "-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-shared-libsan",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]

    def one(src):
        obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
        r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", *flags, "-c", src, "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc (sanitized host build) failed for %s:\n%s" % (src, r.stdout + r.stderr))
        return obj

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC",
                           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                           "-shared-libsan", "-o", SAN_LIB, *objs])
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    build()
