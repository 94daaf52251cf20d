"""Builds libjev.so (HIP kernels + host runtime + C ABI) for gfx950, in-tree.

    python -m shared_prefix_kv_amd.build            # the library
    python -m shared_prefix_kv_amd.build --sanitize # a checking build, host code only

Compiles every source with hipcc and links ``shared_prefix_kv_amd/lib/libjev.so``.
Packed-FP32 instructions are disabled for the device code
(``-target-feature -packed-fp32-ops``); hipcc's host pass warns that it does
not know that feature, which is harmless.

``--sanitize`` builds ``_build/sanitize/libjev.so`` with AddressSanitizer and
UndefinedBehaviorSanitizer on the host code (the device code is built as
usual).  It is never loaded by the product path; the CPU tests run against it
with::

    JEV_LIB=_build/sanitize/libjev.so \
    LD_PRELOAD=$(python -m shared_prefix_kv_amd.build --asan-runtime) \
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1 \
    python -m pytest tests -m "not gpu"
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


SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _compile(src: str, obj_dir: str = OBJ_DIR, extra=()) -> str:
    base = os.path.splitext(os.path.basename(src))[0]
    obj = os.path.join(obj_dir, base + ".o")
    lang = [] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [HIPCC] + COMMON + list(extra) + lang + ["-c", src, "-o", obj]
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


def build_sanitized(verbose: bool = False) -> str:
    """The checking build: host code with ASan + UBSan, into _build/sanitize."""
    out_dir = os.path.join(OBJ_DIR, "sanitize")
    os.makedirs(out_dir, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, out_dir, SANITIZE), SOURCES))
    lib = os.path.join(out_dir, "libjev.so")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", lib] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    if verbose:
        print("built", lib)
    return lib


def asan_runtime() -> str:
    """The compiler's shared AddressSanitizer runtime (to preload into python)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        res = subprocess.run([HIPCC, "-print-resource-dir"], stdout=subprocess.PIPE, text=True).stdout.strip()
        path = os.path.join(res, "lib", "linux", "libclang_rt.asan-x86_64.so")
    return path


if __name__ == "__main__":
    if "--asan-runtime" in sys.argv:
        print(asan_runtime())
    elif "--sanitize" in sys.argv:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
