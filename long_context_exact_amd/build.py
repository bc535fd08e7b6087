"""Builds libdfa.so in-tree with hipcc for gfx950.

    python -m long_context_exact_amd.build      # or __graft_entry__.build()

Every source under csrc/ is compiled to an object in csrc/../_build and the
objects are linked into long_context_exact_amd/lib/libdfa.so.  All device
code is compiled with the packed-fp32 instruction feature turned off.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_DIR = os.path.join(PKG, "lib")
# DFA_LIBRARY selects another build of the same sources (the host-sanitized
# one, for the CPU tests); by default the product library.
LIB_PATH = os.environ.get("DFA_LIBRARY") or os.path.join(LIB_DIR, "libdfa.so")
SANITIZED_LIB_PATH = os.path.join(LIB_DIR, "libdfa_hostsan.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-source compiler options, each measured on its kernel: the forward and
# dK/dV schedule best with the ILP-maximising machine scheduler (about 2.5 %
# and 1 % faster), dQ with the AMDGPU register-pressure trackers (about 6 %).
FILE_FLAGS = {"fwd_mfma.hip": ["-mllvm", "--amdgpu-sched-strategy=max-ilp"],
              "dkdv_mfma.hip": ["-mllvm", "--amdgpu-sched-strategy=max-ilp"],
              "dq_mfma.hip": ["-mllvm", "--amdgpu-use-amdgpu-trackers"]}


def _sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src,
           "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{out}")
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def build_host_sanitized(jobs: int | None = None) -> str:
    """Every source built with AddressSanitizer and UndefinedBehaviorSanitizer
    on its host code only (the device code is built unsanitized, at -O1, and
    never run from this library), linked into lib/libdfa_hostsan.so.  It runs
    the schedules, the argument checks and the workspace sizing exactly as
    the product library does, for the CPU tests to drive under the
    sanitizers.  Returns its path."""
    out_dir = os.path.join(BUILD_DIR, "hostsan")
    os.makedirs(out_dir, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC",
             f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def one(src):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        res = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True,
                             text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc (host sanitized) failed on {src}:\n{res.stderr}")
        return obj

    srcs = _sources()
    with cf.ThreadPoolExecutor(jobs or min(len(srcs), 8)) as ex:
        objs = list(ex.map(one, srcs))
    tmp = SANITIZED_LIB_PATH + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Xarch_host",
           "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", *objs,
           "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, SANITIZED_LIB_PATH)
    return SANITIZED_LIB_PATH


def sanitizer_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (to preload into
    an uninstrumented python that loads the sanitized library)."""
    res = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    return res.stdout.strip()


def build(extra_flags=(), jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source and link libdfa.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    srcs = _sources()
    jobs = jobs or min(len(srcs), 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), srcs))
    product = os.path.join(LIB_DIR, "libdfa.so")
    tmp = product + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, product)
    if verbose:
        print(f"built {product}")
    return product


if __name__ == "__main__":
    build(verbose=True)
