"""Builds ``_build_san/libwf_san.so``: the same library with its host code
(plan, validation, runtime, bindings of the C ABI) compiled under
AddressSanitizer and UndefinedBehaviorSanitizer.  Device code is compiled as
usual (no GPU sanitizer).  Used by ``tests/test_abi_sanitized.py``, which
runs the C-ABI CPU tests against it with the sanitizer runtime preloaded.

Usage: ``python -m chunk_causal_dit_round_amd.build_sanitized``.
"""

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

from .build import CSRC, CXX_SOURCES, FILE_FLAGS, HIP_FLAGS, HIP_SOURCES, INCLUDE, PKG, _hipcc, _run

BUILD_SAN = os.path.join(PKG, "_build_san")
LIB_SAN = os.path.join(BUILD_SAN, "libwf_san.so")
LLVM_BIN = "/opt/rocm/llvm/bin"

# Host-side sanitizers only: each flag follows -Xarch_host.
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of clang's AddressSanitizer runtime (to preload into Python)."""
    out = subprocess.run([os.path.join(LLVM_BIN, "clang++"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True).stdout.strip()
    if out and os.path.isabs(out) and os.path.exists(out):
        return out
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not hits:
        raise RuntimeError("AddressSanitizer runtime not found")
    return hits[0]


def build_sanitized(verbose: bool = False) -> str:
    os.makedirs(BUILD_SAN, exist_ok=True)
    hipcc = _hipcc()
    flags = [f for f in HIP_FLAGS if f != "-O3"] + ["-O1", "-g"]
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_SAN, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        jobs.append([hipcc, *flags, *FILE_FLAGS.get(src, []), *HOST_SAN, "-I", INCLUDE, "-I", CSRC,
                     *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD_SAN, src + ".o")
        jobs.append([os.path.join(LLVM_BIN, "clang++"), "-O1", "-g", "-std=c++17", "-fPIC", "-Wall",
                     "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                     "-fno-omit-frame-pointer", "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    objs = [j[-1] for j in jobs]
    tmp = LIB_SAN + ".tmp"
    _run([hipcc, f"--offload-arch=gfx950", "-shared", "-fPIC", "-fno-gpu-sanitize",
          "-fsanitize=address,undefined", *objs, "-o", tmp, "-L/opt/rocm/lib", "-lhipblaslt"], verbose)
    os.replace(tmp, LIB_SAN)
    return LIB_SAN


if __name__ == "__main__":
    print(build_sanitized(verbose=True))
