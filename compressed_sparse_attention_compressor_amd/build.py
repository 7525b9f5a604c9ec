"""Builds libcsa.so (HIP, gfx950 only) in the package directory.

Usage: python -m compressed_sparse_attention_compressor_amd.build
Every call recompiles every source (no stale objects are ever reused).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcsa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    "-I" + os.path.join(ROOT, "include"),
]
SOURCES = ["abi.hip", "compress.hip", "compress_hidden.hip", "index.hip", "topk.hip", "pool.hip", "swa.hip", "attn.hip"]
# The indexer folds every MFMA result through ReLU and the head weights on
# the vector unit: results written to AGPRs would each need a copy first.
# Attention has no NaN inputs or intermediates by construction (masked logits
# are -inf, never NaN): without NaN semantics a float max needs no operand
# quieting first and folds with its DPP source.
EXTRA = {"index.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "attn.hip": ["-fno-honor-nans"]}


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    if os.path.isdir(OBJ):
        shutil.rmtree(OBJ)
    os.makedirs(OBJ)
    workers = min(len(SOURCES), max(1, (os.cpu_count() or 2) // 2))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


# Sanitized build: the host code (argument checks,
# workspace sizing, dispatch) instrumented with AddressSanitizer and
# UndefinedBehaviorSanitizer (the device code is built as usual, never run
# by the CPU ABI tests, which never reach a launch).  The sanitizer flags go to the host pass
# only (-Xarch_host before each); the link is a plain clang++ line.
CLANGXX = os.environ.get("CLANGXX", "/opt/rocm/llvm/bin/clang++")
SAN_COMPILE = ["-O1", "-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all"]
SAN_LINK = ["-fsanitize=address,undefined", "-shared-libasan"]


def build_host_sanitized(out_dir: str) -> str:
    """Builds the sanitized host-only libcsa.so into out_dir; returns its path."""
    os.makedirs(out_dir, exist_ok=True)

    def one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *SAN_COMPILE, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"host-only compile failed on {src}:\n{r.stderr}")
        return obj

    workers = min(len(SOURCES), max(1, (os.cpu_count() or 2) // 2))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(one, SOURCES))
    out = os.path.join(out_dir, "libcsa_san.so")
    link = [CLANGXX, "-shared", "-fPIC", *objs, *SAN_LINK, "-L/opt/rocm/lib", "-lamdhip64", "-o", out]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitized link failed:\n" + r.stderr)
    return out


if __name__ == "__main__":
    build()
    sys.exit(0)
