"""Compiles the HIP sources into the in-tree shared library ``libjt.so``.

hipcc cross-compiles for gfx950 on a machine without a GPU.  Object files go
to ``_build/`` next to this file; the library lands next to this file.

``build_host_sanitized()`` (``python -m tree_causal_attention_amd.build
--host-sanitize``) builds ``libjt_hostsan.so``: the same sources with the host
code instrumented by AddressSanitizer and UndefinedBehaviorSanitizer (the
device code is compiled as usual and not instrumented).  It serves the C
ABI's argument validation checks on a machine without a GPU; see
``tests/test_host_sanitized_abi.py``.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libjt.so")
SAN_OBJ = os.path.join(OBJ, "hostsan")
SAN_LIB = os.path.join(HERE, "libjt_hostsan.so")
CLANGXX = os.environ.get("JT_CLANGXX", "/opt/rocm/lib/llvm/bin/clang++")
SOURCES = ["api.hip", "build_tree.hip", "tree_meta.hip", "tree_attention.hip", "accept.hip",
           "commit.hip", "stochastic.hip", "draft_scan.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 VALU ops stay off (see the design notes on MI355X traps)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return out


def build(jobs: int = 8) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# sanitizers on the host code only (each flag after -Xarch_host).  The device
# code is never launched by the checks this library serves: the draft scan's
# many unrolled instances are left unoptimised so that they compile in seconds
# (the attention's inline assembly needs its operands placed, so -O1 there).
SAN_DEVICE_OPT = {"draft_scan.hip": "-O0"}
SAN_FLAGS = [
    "--offload-arch=gfx950", "-Xarch_host", "-O1", "-Xarch_host", "-g",
    "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
]


def _compile_san(src: str) -> str:
    out = os.path.join(SAN_OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, SAN_DEVICE_OPT.get(src, "-O1"), *SAN_FLAGS, "-c", os.path.join(CSRC, src),
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc (host, sanitized) failed on {src}:\n{r.stdout}\n{r.stderr}")
    return out


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to preload into Python)."""
    r = subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    return r.stdout.strip()


def build_host_sanitized(jobs: int = 8) -> str:
    os.makedirs(SAN_OBJ, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(_compile_san, SOURCES))
    tmp = SAN_LIB + ".tmp"
    # linked by the host compiler against the shared sanitizer runtimes
    link = [CLANGXX, "-shared", "-fPIC", "-shared-libsan", "-fsanitize=address,undefined",
            "-o", tmp, *objs, "-L/opt/rocm/lib", "-lamdhip64",
            "-Wl,-rpath," + os.path.dirname(asan_runtime())]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--host-sanitize" in sys.argv[1:]:
        print(build_host_sanitized())
    else:
        print(build())
    sys.exit(0)
