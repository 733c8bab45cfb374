"""Build libkla.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python bius_scan_sequence_amd/build.py

Every call recompiles.  Objects go to bius_scan_sequence_amd/_build/, the
library to bius_scan_sequence_amd/libkla.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkla.so")
SOURCES = ["kla_forward.hip", "kla_forward_run.hip", "kla_precision.hip", "kla_decode.hip", "kla_backward.hip", "kla_vprec.hip", "kla_util.hip", "kla_api.hip"]
ARCH = os.environ.get("KLA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm under /opt/rocm)")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
        # packed fp32 instructions are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wno-unused-command-line-argument",
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


# Host-sanitizer build: the C ABI's host code (argument validation, workspace
# layout, launch set-up in kla_api.hip) compiled with AddressSanitizer and
# UBSan for the host side only; every kernel object is the ordinary one.  The
# library expects the ASan runtime preloaded (see asan_runtime()).
SAN_DIR = os.path.join(BUILD, "hostsan")
SAN_LIB = os.path.join(SAN_DIR, "libkla_hostsan.so")


def asan_runtime() -> str:
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    return subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True, check=True).stdout.strip()


def build_host_sanitized(verbose: bool = False) -> str:
    """Builds SAN_LIB, reusing the ordinary kernel objects when they exist."""
    if not all(os.path.exists(os.path.join(BUILD, os.path.splitext(s)[0] + ".o")) for s in SOURCES):
        build()
    os.makedirs(SAN_DIR, exist_ok=True)
    obj = os.path.join(SAN_DIR, "kla_api_san.o")
    cmd = [hipcc(), *common_flags(), "-g", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-c", os.path.join(CSRC, "kla_api.hip"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    objs = [obj] + [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "kla_api.hip"]
    cmd = ["g++", "-shared", "-fPIC", "-o", SAN_LIB, *objs, "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib", "-Wl,--allow-shlib-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


# Timeline build: the forward kernels and the backward compiled with
# -DKLA_TIMELINE (per workgroup real-time stamps of the run-streaming and the
# segmented forward, per wave phase sums of the backward chunk kernel, read by
# bius_scan_sequence_amd/timeline.py); every other object is the ordinary one.
TL_DIR = os.path.join(BUILD, "timeline")
TL_LIB = os.path.join(PKG, "libkla_timeline.so")


def build_timeline(verbose: bool = False) -> str:
    """Builds TL_LIB next to libkla.so, reusing the ordinary objects when they exist."""
    if not all(os.path.exists(os.path.join(BUILD, os.path.splitext(s)[0] + ".o")) for s in SOURCES):
        build()
    os.makedirs(TL_DIR, exist_ok=True)
    traced = ("kla_forward_run.hip", "kla_forward.hip", "kla_backward.hip")
    objs = []
    for src in traced:
        obj = os.path.join(TL_DIR, os.path.splitext(src)[0] + "_tl.o")
        cmd = [hipcc(), *common_flags(), "-DKLA_TIMELINE", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        objs.append(obj)
    objs += [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s not in traced]
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", TL_LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print("built", TL_LIB)
    return TL_LIB


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        build_host_sanitized(verbose=True)
    elif "--timeline" in sys.argv:
        build_timeline(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
