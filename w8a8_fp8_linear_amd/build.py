"""Build libw8a8.so for gfx950 with hipcc (``python -m w8a8_fp8_linear_amd.build``).

One shared library, compiled in-tree next to this file. Flags: gfx950 only,
-O3, and packed-fp32 instruction selection switched off for device code.

``build(out=..., sanitize_host=True)`` builds a copy whose host code (the
C ABI's argument checks, workspace layout and launch set-up) carries
AddressSanitizer and UndefinedBehaviorSanitizer; device code is unchanged.
Load it with the sanitizer runtime preloaded (``sanitizer_runtime()``) and
``W8A8_LIB`` pointing at it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["api.hip", "quant.hip", "gemm.hip", "w8a16.hip", "moe.hip", "mx.hip"]
OUT = os.path.join(HERE, "libw8a8.so")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# each sanitizer flag applies to the host pass only
SANITIZE_HOST = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
]


def sanitizer_runtime() -> str:
    """The shared AddressSanitizer runtime of the compiler hipcc drives (it
    also carries UBSan's handlers); a process loading a host-sanitized build
    must preload it."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found")
    return path


def build(verbose: bool = False, out: str = OUT, sanitize_host: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, *(SANITIZE_HOST if sanitize_host else []), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
