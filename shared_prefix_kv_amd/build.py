"""Builds libjev.so (HIP kernels + host runtime + C ABI) for gfx950, in-tree.

    python -m shared_prefix_kv_amd.build

Compiles every source with hipcc and links ``shared_prefix_kv_amd/lib/libjev.so``.
Packed-FP32 instructions are disabled for the device code
(``-target-feature -packed-fp32-ops``); hipcc's host pass warns that it does
not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "lib")
LIB = os.path.join(OUT_DIR, "libjev.so")
OBJ_DIR = os.path.join(ROOT, "_build")

SOURCES = [
    os.path.join(CSRC, "kernels", "kernels.hip"),
    os.path.join(CSRC, "kernels", "gemm.hip"),
    os.path.join(CSRC, "host", "tree.cpp"),
    os.path.join(CSRC, "host", "answers.cpp"),
    os.path.join(CSRC, "host", "api.cpp"),
]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wno-unused-result"]


def _compile(src: str) -> str:
    base = os.path.splitext(os.path.basename(src))[0]
    obj = os.path.join(OBJ_DIR, base + ".o")
    lang = [] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [HIPCC] + COMMON + lang + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in r.stdout.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
