"""Build the HIP library librelbias_attn.so for gfx950 (in-tree, with hipcc).

Usage: python -m transformer_attention_learned_amd.build   (or build_library()).
Compiles every source under csrc/ with hipcc --offload-arch=gfx950 and links
one shared library next to this file.  A GPU is not needed to build.
"""

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
LIB = os.path.join(PKG, "librelbias_attn.so")

SOURCES = ["api.cpp", "launch_attr.cpp", "fwd_bf16.hip", "fwd_bf16_split.hip", "attn_f32.hip",
           "decode_bf16.hip", "bwd_bf16.hip", "bwd_f32.hip", "kv_fp4.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            # no packed-fp32 VALU instructions in device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA accumulators in architectural VGPRs (the softmax rescales them with VALU ops)
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", out] + _flags()
    if src.endswith(".cpp"):
        cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", out] + _flags()
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    return out


def build_library(verbose: bool = False) -> str:
    """Compile all sources and link librelbias_attn.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


# Host-only translation units (argument validation, dispatch, per-device state): the sanitizer
# build instruments these with AddressSanitizer and UndefinedBehaviorSanitizer.
HOST_SOURCES = ["api.cpp", "launch_attr.cpp"]
SAN_LIB = os.path.join(BUILD, "san", "librelbias_attn_san.so")


def sanitizer_runtime() -> str:
    """clang's shared AddressSanitizer runtime (it has to be preloaded into the host process)."""
    import glob
    cands = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(hipcc())), "llvm", "lib",
                                          "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not cands:
        raise RuntimeError("clang's libclang_rt.asan-x86_64.so not found under the ROCm tree")
    return cands[-1]


def build_sanitized(verbose: bool = False) -> str:
    """A copy of the library whose host code (HOST_SOURCES) is built with -fsanitize=address and
    -fsanitize=undefined (host pass only), linked with the ordinary kernel objects; for the
    CPU-tier validation tests.  Builds the ordinary objects first if they are missing."""
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    dev_objs = [os.path.join(BUILD, s + ".o") for s in SOURCES if s not in HOST_SOURCES]
    if not all(os.path.exists(o) for o in dev_objs):
        build_library(verbose)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
    objs = []
    for src in HOST_SOURCES:
        out = os.path.join(BUILD, "san", src + ".o")
        cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", out] + _flags() + san
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized compile of {src} failed:\n{r.stdout}{r.stderr}")
        objs.append(out)
    clangxx = os.path.join(os.path.dirname(os.path.dirname(hipcc())), "llvm", "bin", "clang++")
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(hipcc())), "lib")
    cmd = [clangxx, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan", "-o",
           SAN_LIB + ".tmp"] + objs + dev_objs + ["-L", rocm_lib, "-lamdhip64",
                                                  "-Wl,-rpath," + rocm_lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitized link failed:\n" + r.stdout + r.stderr)
    os.replace(SAN_LIB + ".tmp", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
