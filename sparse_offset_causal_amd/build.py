"""Build libsoc_attn.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsoc_attn.so")

SOURCES = ["abi.cpp", "prefill_bf16.hip", "decode_bf16.hip", "attn_f32.hip", "blocksel.hip", "ring.hip", "mla_bf16.hip", "dsa_bf16.hip"]

# Packed fp32 VALU ops are turned off for device code (the host pass ignores the feature).
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]
# Kernel sources only: no kernel reads or produces NaN on purpose, so min/max need no NaN
# quieting; infinities keep their IEEE meaning.  The host-side argument checks (abi.cpp,
# which tests for NaN) are compiled without these.
KERNEL_FLAGS = ["-fno-honor-nans", "-mno-amdgpu-ieee"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    extra = KERNEL_FLAGS if src.endswith(".hip") else []
    cmd = [hipcc(), *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if warn and verbose:
        print(warn, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


SANITIZED_LIB = os.path.join(BUILD, "libsoc_attn_asan.so")


def build_sanitized(verbose: bool = False) -> str:
    """The same library with its host code (the C ABI layer) built under AddressSanitizer and
    UndefinedBehaviorSanitizer (device code unchanged: the sanitizers apply to the host pass
    only), for running the argument-checking tests on the CPU.  Load it with the ASan runtime
    preloaded (sanitizer_runtime()).  Written to _build/, never loaded by the package itself."""
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    abi_obj = os.path.join(BUILD, "abi_asan.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
           "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    cmd = [hipcc(), *FLAGS, *san, "-x", "hip", "-c", os.path.join(CSRC, "abi.cpp"), "-o", abi_obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on abi.cpp (sanitized):\n{r.stdout}\n{r.stderr}")
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
           "-fsanitize=undefined", "-shared-libsan", abi_obj, *objs, "-o", SANITIZED_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed (sanitized):\n{r.stdout}\n{r.stderr}")
    return SANITIZED_LIB


def sanitizer_runtime() -> str:
    """Path of the ASan runtime (which carries the UBSan handlers) to preload into Python."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


if __name__ == "__main__":
    if "sanitized" in sys.argv[1:]:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
