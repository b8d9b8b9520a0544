"""Builds libdflash2.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Usage: python -m block_draft_head_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdflash2.so")
SOURCES = ["api.cpp", "conv.hip", "lmhead.hip", "proj.hip", "selector.hip", "selector_bwd.hip"]

ARCH = os.environ.get("DFLASH2_OFFLOAD_ARCH", "gfx950")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-result",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the DFlash2 library)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if warn:
        print(f"[{src}]\n{warn}", file=sys.stderr)
    return obj


def build(jobs: int = 8, verbose: bool = True) -> str:
    """Compile every source and link the shared library.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host code instrumented by AddressSanitizer and UndefinedBehaviorSanitizer;
# device code left alone (each flag goes to the host compilation only).
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan"]


def asan_runtime() -> str:
    """The compiler's shared AddressSanitizer runtime (LD_PRELOAD it into a
    process that loads the sanitized library)."""
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang++")
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime was not found")
    return path


def build_host_sanitized(out_dir: str, jobs: int = 8) -> str:
    """The same sources as build(), at -O1, with the host side sanitized: a
    library for the ABI tests' host validation on a machine without a GPU.
    Its kernels are never launched.  Returns the library path."""
    os.makedirs(out_dir, exist_ok=True)
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-fno-omit-frame-pointer", *SANITIZE]

    def one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), "-x", "hip", *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(one, SOURCES))
    lib = os.path.join(out_dir, "libdflash2.so")
    rt_dir = os.path.dirname(asan_runtime())
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *SANITIZE, f"-Wl,-rpath,{rt_dir}", "-o", lib, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stderr}")
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    build(ap.parse_args().jobs)
