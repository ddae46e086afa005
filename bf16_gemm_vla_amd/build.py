"""Build the gfx950 HIP library in-tree: bf16_gemm_vla_amd/libvla.so.

    python -m bf16_gemm_vla_amd.build

Every HIP translation unit is compiled with hipcc for gfx950 only, with
packed-fp32 instruction generation disabled, then linked into one shared
library exporting the C ABI declared in include/vla.h.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libvla.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["codec.hip", "gemm.hip", "gemm_wide.hip", "chain.hip", "boundary.hip", "probe.hip", "abi.cpp"]
HIPFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer for the checking
# build (libvla_san.so): only the host pass is instrumented; the library is
# linked without a sanitizer runtime, which the process preloads.
SAN_OBJDIR = os.path.join(ROOT, "_build_san")
SAN_LIB = os.path.join(PKG, "libvla_san.so")
HOST_SANITIZE = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
]


def _compile(src: str, sanitize: bool = False) -> str:
    objdir = SAN_OBJDIR if sanitize else OBJDIR
    os.makedirs(objdir, exist_ok=True)
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *HIPFLAGS, *(HOST_SANITIZE if sanitize else []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(sanitize: bool = False) -> str:
    """Compile and link libvla.so; with sanitize, the host-instrumented
    checking build libvla_san.so instead (the product never loads it)."""
    lib = SAN_LIB if sanitize else LIB
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    # A kernel template whose body the host pass cannot instantiate loses its
    # launch stub without a diagnostic; the library would then fail to load.
    # Refuse to install a library with undefined symbols of its own.
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    own = [l.split()[-1] for l in nm.stdout.splitlines() if "_ZN3vla" in l]
    if nm.returncode != 0 or own:
        os.remove(tmp)
        raise RuntimeError(os.path.basename(lib) + " has undefined symbols of its own: " + ", ".join(own[:8]))
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build())
