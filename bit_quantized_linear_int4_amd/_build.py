"""Builds libwq.so (every HIP source for gfx950) in-tree.

Usage: ``python -m bit_quantized_linear_int4_amd._build`` or
``__graft_entry__.build()``.  Objects go to ``_build/`` at the repository
root; the shared library lands next to this file.  With ``--sanitized`` a
second library whose host-side C-ABI layer carries AddressSanitizer and
UndefinedBehaviorSanitizer is built at ``_build/sanitized/libwq.so``.
"""

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libwq.so")
ARCH = "gfx950"


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libwq)")


# -packed-fp32-ops: no v_pk_*_f32 in generated code.
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-x", "hip",
    "-I", INCLUDE, "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src):
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


# The host-side C-ABI layer: argument checks, launch plans, codebooks.
HOST_SOURCES = ("wq_api.cpp", "nf4_levels.cpp")
SANITIZED_DIR = os.path.join(OBJDIR, "sanitized")
# AddressSanitizer and UndefinedBehaviorSanitizer on the host code only
# (-Xarch_host before each flag); the device code is built as usual.
SANITIZE = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
            "-Xarch_host -fno-omit-frame-pointer").split()


def sanitizer_runtime():
    """The clang ASan runtime hipcc's sanitized code links against (to
    LD_PRELOAD into a Python process that loads the sanitized library)."""
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm")
    found = sorted(glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang ASan runtime not found")
    return found[-1]


def build_host_sanitized(verbose=False):
    """A second libwq.so whose host-side C-ABI layer carries ASan and UBSan,
    linked with the regular kernel objects, at _build/sanitized/libwq.so.
    Load it through WQ_LIBRARY with the ASan runtime preloaded; only host
    code paths (argument checks) are meant to run under it."""
    os.makedirs(SANITIZED_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    objs = []
    for src in srcs:
        name = os.path.basename(src)
        if name in HOST_SOURCES:
            obj = os.path.join(SANITIZED_DIR, name + ".o")
            cmd = [hipcc()] + COMMON + ["-g"] + SANITIZE + ["-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        else:
            obj = os.path.join(OBJDIR, name + ".o")
            if not os.path.exists(obj):
                obj = _compile(src)
        objs.append(obj)
    lib = os.path.join(SANITIZED_DIR, "libwq.so")
    cmd = ([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + SANITIZE +
           ["-shared-libsan", "-o", lib] + objs)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {lib} (host code with ASan and UBSan)")
    return lib


if __name__ == "__main__":
    build(verbose=True)
    if "--sanitized" in sys.argv:
        build_host_sanitized(verbose=True)
    sys.exit(0)
