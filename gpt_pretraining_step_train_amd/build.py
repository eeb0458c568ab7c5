"""Build libgptmi.so (HIP kernels + C ABI) for gfx950 with hipcc, in place."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libgptmi.so")
SOURCES = ["gemm.hip", "elementwise.hip", "attention.hip", "gpt.hip"]
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off (the compiler would otherwise form them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, objdir: str) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 4)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the C ABI (gpt.hip),
# linked with the ordinary objects of the kernel files; device code is built as usual
SAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that a host process preloads for the sanitized build."""
    import glob
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang", "*", "lib",
                                         "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under the ROCm llvm tree")
    return hits[-1]


def build_host_sanitized() -> str:
    objdir = os.path.join(HERE, "_build")
    others = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "gpt.hip"]
    if not all(os.path.exists(o) for o in others):
        build()
    sdir = os.path.join(objdir, "sanitized")
    os.makedirs(sdir, exist_ok=True)
    obj = os.path.join(sdir, "gpt.o")
    flags = [f for f in FLAGS if f != "-O3"] + SAN_FLAGS
    r = subprocess.run([HIPCC, *flags, "-c", os.path.join(CSRC, "gpt.hip"), "-o", obj], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the sanitized gpt.hip:\n{r.stderr[-6000:]}")
    lib = os.path.join(sdir, "libgptmi_sanitized.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", "-o", lib, obj, *others], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr[-6000:]}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
