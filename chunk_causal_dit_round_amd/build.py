"""Builds ``libwf.so`` (HIP kernels + C ABI) in-tree for gfx950.

Usage: ``python -m chunk_causal_dit_round_amd.build`` or ``build_library()``.
Always recompiles.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libwf.so")
ARCH = "gfx950"

HIP_SOURCES = ["wf_runtime.cpp", "wf_publish.hip", "wf_attention.hip", "wf_attention_fp8.hip",
               "wf_attention_fp8k.hip", "wf_dit.hip", "wf_dit.cpp"]
# Attention scores are finite or -inf, never NaN: without NaN semantics the
# row max needs no canonicalising v_max x,x per score.
FILE_FLAGS = {"wf_attention.hip": ["-fno-honor-nans"],
              "wf_attention_fp8.hip": ["-fno-honor-nans"],
              "wf_attention_fp8k.hip": ["-fno-honor-nans"]}
CXX_SOURCES = ["wf_plan.cpp"]

# Packed fp32 VALU forms are switched off for all device code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-command-line-argument"]


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)


def build_library(verbose: bool = False) -> str:
    """Compile every source and link ``libwf.so``; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC,
              "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        _run([hipcc, *HIP_FLAGS, *FILE_FLAGS.get(src, []), "-I", INCLUDE, "-I", CSRC, *lang,
              "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    # the DiT block's products go through hipBLASLt (the process's copy of
    # libhipblaslt.so.1: PyTorch's own when loaded from Python)
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
          "-L/opt/rocm/lib", "-lhipblaslt"], verbose)
    os.replace(tmp, LIB)
    return LIB
