"""Build libflexattn.so in-tree with hipcc for gfx950.

    python -m attention_tiled_attn_amd.build [-v] [--define NAME=VALUE ...]
    python -m attention_tiled_attn_amd.build --sanitize

Every call recompiles (sources are few). Objects go to _build/ beside this
file; the shared library is written next to this file. --define passes a
preprocessor definition to every source (the kernels' build options, e.g.
FLEXATTN_EXP2_POLY_CHUNKS=2 for the software-exp2 A/B).

--sanitize builds libflexattn_san.so instead: the C ABI's host code
(api.cpp) compiled by the host C++ compiler with the address and
undefined-behaviour sanitizers, linked with stand-ins for the kernels and
HIP calls (csrc/host_stubs.cpp). It runs the argument checks only, on the
CPU (tests/test_abi_sanitized.py loads it with the sanitizer runtime
preloaded).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libflexattn.so")
ARCH = "gfx950"

SOURCES = ["attn_fwd.hip", "attn_fwd_pp.hip", "attn_bwd.hip", "block_mask.hip", "api.cpp"]
# microbenchmarks of the units the kernels use (measurement tooling, its own
# library; attention_tiled_attn_amd.microbench runs them)
MB_SOURCE = "microbench.hip"
MB_OUT = os.path.join(HERE, "libflexattn_mb.so")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Wall", "-Wno-unused-function",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build the library)")
    return path


def _compile(src: str, obj: str, verbose: bool, defines=()) -> None:
    cmd = [hipcc(), *COMMON, *(f"-D{d}" for d in defines), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)


def _link(objs, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, defines=()) -> str:
    """Build libflexattn.so (returned) and the microbenchmark library
    libflexattn_mb.so beside it."""
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    srcs = SOURCES + [MB_SOURCE]
    objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        list(ex.map(lambda a: _compile(a[0], a[1], verbose, defines), zip(srcs, objs)))
    _link(objs[:-1], OUT, verbose)
    _link(objs[-1:], MB_OUT, verbose)
    return OUT


SAN_OUT = os.path.join(HERE, "libflexattn_san.so")
SAN_FLAGS = ["-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def build_sanitized(verbose: bool = False) -> str:
    cxx = shutil.which("g++") or shutil.which("c++")
    if not cxx:
        raise RuntimeError("no host C++ compiler for the sanitizer build")
    rocm_inc = os.path.join(os.path.dirname(os.path.dirname(hipcc())), "include")
    tmp = SAN_OUT + ".tmp"
    cmd = [cxx, *SAN_FLAGS, f"-I{rocm_inc}", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "host_stubs.cpp"), "-shared", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer build failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_OUT)
    return SAN_OUT


if __name__ == "__main__":
    args = sys.argv[1:]
    defs = [args[i + 1] for i, a in enumerate(args) if a == "--define" and i + 1 < len(args)]
    if "--sanitize" in args:
        print(build_sanitized(verbose="-v" in args))
    else:
        print(build(verbose="-v" in args, defines=defs))
