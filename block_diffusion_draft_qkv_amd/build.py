"""Build ``libdflash.so`` (the C-ABI library of include/dflash.h) for gfx950.

Every HIP source under ``csrc/`` is compiled with hipcc for gfx950 only and
linked into one shared library next to this file. Packed fp32 VALU ops are
turned off for the device code (``-packed-fp32-ops``); the host pass of hipcc
warns that it does not know that feature, which is harmless. MFMA results are
kept in ordinary VGPRs (``-amdgpu-mfma-vgpr-form``) so that the online-softmax
rescale of the accumulators needs no AGPR moves.

``build(sanitize=True)`` instead compiles the same sources with
AddressSanitizer and UndefinedBehaviorSanitizer on the host code only
(``-Xarch_host`` before each ``-fsanitize=``; the device code is unchanged) into
the static archive ``_build/sanitize/libdflash_san.a``, for a host-only check
program that links it with a host stand-in of the HIP runtime.

Usage: ``python -m block_diffusion_draft_qkv_amd.build [--debug] [--sanitize]``.
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
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdflash.so")
ARCH = "gfx950"
SOURCES = ["gemm.hip", "norm_rope_append.hip", "attention.hip", "row_norm.hip", "dflash.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the DFlash kernels)")


def flags(debug: bool = False):
    f = ["-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-Wno-unused-command-line-argument"]
    f += ["-O1", "-g"] if debug else ["-O3"]
    return f


SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LIB = os.path.join(PKG, "_build", "sanitize", "libdflash_san.a")


def build(debug: bool = False, verbose: bool = False, sanitize: bool = False) -> str:
    cc = hipcc()
    out_dir = os.path.join(PKG, "_build", "sanitize") if sanitize else os.path.join(PKG, "_build")
    os.makedirs(out_dir, exist_ok=True)
    extra = [*SANITIZE_FLAGS, "-O1", "-g"] if sanitize else []

    def compile_one(src: str) -> str:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *flags(debug), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd.insert(1, "-xhip")
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    if sanitize:
        tmp = SAN_LIB + ".tmp"
        if os.path.exists(tmp):
            os.remove(tmp)
        r = subprocess.run(["ar", "rcs", tmp, *objs], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"ar failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, SAN_LIB)
        return SAN_LIB
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--debug", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--sanitize", action="store_true")
    a = ap.parse_args()
    print(build(debug=a.debug, verbose=a.verbose, sanitize=a.sanitize))
    sys.exit(0)
