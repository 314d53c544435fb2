"""Build the host-only ABI check: the library's sources compiled with
AddressSanitizer and UndefinedBehaviorSanitizer on their host code
(``build(sanitize=True)``), linked with the host stand-in of the HIP runtime
(hip_stub.cpp) and the check program (abi_host_check.cpp) into one executable,
so that the sanitizer runtime is the program's own (no preloading) and no GPU
runtime is involved. Test infrastructure: nothing here is part of the library.

Usage: ``python tests/host_abi/build_check.py`` prints the executable's path.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "_build")
EXE = os.path.join(OUT, "abi_host_check")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _sources():
    sys.path.insert(0, ROOT)
    from block_diffusion_draft_qkv_amd import build as b
    srcs = [os.path.join(b.CSRC, s) for s in b.SOURCES]
    srcs += [os.path.join(b.CSRC, f) for f in sorted(os.listdir(b.CSRC)) if f.endswith(".h")]
    srcs += [os.path.join(b.INCLUDE, f) for f in sorted(os.listdir(b.INCLUDE))]
    srcs += [os.path.join(HERE, f) for f in ("hip_stub.cpp", "hip_stub.h", "abi_host_check.cpp", "plan_check.cpp",
                                             "build_check.py")]
    srcs.append(os.path.abspath(b.__file__))
    return b, srcs


def build_check(force: bool = False) -> str:
    """Build (when a source changed since the last build) and return the path
    of the check executable."""
    b, srcs = _sources()
    h = hashlib.sha256()
    for p in srcs:
        with open(p, "rb") as f:
            h.update(p.encode() + b"\0" + f.read())
    stamp = os.path.join(OUT, "sources.sha256")
    digest = h.hexdigest()
    if not force and os.path.exists(EXE) and os.path.exists(stamp) and open(stamp).read() == digest:
        return EXE
    os.makedirs(OUT, exist_ok=True)
    lib = b.build(sanitize=True)
    objs = []
    for src, extra in (("hip_stub.cpp", ["-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include"]),
                       ("abi_host_check.cpp", ["-I", b.INCLUDE])):
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        cmd = [CLANG, "-std=c++17", "-O1", "-g", *SAN, *extra, "-I", HERE, "-c", os.path.join(HERE, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
        objs.append(obj)
    # the plan checker reads the library's kernel argument structs: HIP host code
    obj = os.path.join(OUT, "plan_check.o")
    cmd = [b.hipcc(), "-xhip", "--cuda-host-only", "-std=c++17", "-O1", "-g", *b.SANITIZE_FLAGS, "-I", b.CSRC,
           "-I", b.INCLUDE, "-c", os.path.join(HERE, "plan_check.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling plan_check.cpp failed:\n{r.stdout}\n{r.stderr}")
    objs.append(obj)
    cmd = [CLANG, *SAN, *objs, lib, "-o", EXE + ".tmp", "-lpthread", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking the host check failed:\n{r.stdout}\n{r.stderr}")
    os.replace(EXE + ".tmp", EXE)
    with open(stamp, "w") as f:
        f.write(digest)
    return EXE


if __name__ == "__main__":
    print(build_check(force="--force" in sys.argv))
