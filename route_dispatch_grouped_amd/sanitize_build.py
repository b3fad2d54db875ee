"""Host-sanitizer build of the library, for the CPU test suite.

The C ABI's host code (``csrc/api.cpp``: argument validation, workspace
carving, the per-stream shared-expert bookkeeping, error strings) is compiled
by g++ with AddressSanitizer and UndefinedBehaviorSanitizer and linked with the
kernel objects of the regular hipcc build, which stay uninstrumented.  Only
host code is sanitized; loading the result and running the validation paths
needs no GPU.  The library is loaded into a process that preloads the ASan
runtime (``asan_runtime()``).
"""
from __future__ import annotations

import os
import shutil
import subprocess

from .build import BUILD_DIR, CSRC, INCLUDE, SOURCES, build

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _gxx() -> str:
    g = shutil.which("g++")
    if g is None:
        raise RuntimeError("g++ not found")
    return g


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + r.stdout)


def asan_runtime() -> str:
    """Path of g++'s ASan runtime, to be preloaded into the loading process."""
    out = subprocess.run([_gxx(), "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True, check=True)
    return out.stdout.strip()


def build_sanitized(out_dir: str) -> str:
    """Build ``out_dir/libmoe_mi355x_hostsan.so`` and return its path."""
    kernel_objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in kernel_objs):
        build()
    os.makedirs(out_dir, exist_ok=True)
    gxx = _gxx()
    api_obj = os.path.join(out_dir, "api_hostsan.o")
    _run([gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-Wall", *SANITIZE, "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROCM, "include"), "-I", INCLUDE, "-I", CSRC,
          "-c", os.path.join(CSRC, "api.cpp"), "-o", api_obj])
    lib = os.path.join(out_dir, "libmoe_mi355x_hostsan.so")
    _run([gxx, "-shared", *SANITIZE, "-o", lib, api_obj, *kernel_objs,
          "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    return lib
