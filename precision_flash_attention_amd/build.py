"""Build libsattn.so (HIP kernels + C ABI) for gfx950, in-tree.

hipcc compiles each translation unit for gfx950 only; quant.hip is built with
-ffp-contract=off so that every FP32 step of the quantizer is a single IEEE
operation.  Packed-FP32 VALU instructions are disabled for all device code.

build_host_sanitized(path) builds the same library with AddressSanitizer and
UndefinedBehaviorSanitizer on the host code only (each -fsanitize after
-Xarch_host; device code is built as usual), for the CPU test that drives the
ABI's validation, layout and unpacking paths under the sanitizers.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-std=c++17", "-O3", "-fPIC", "--offload-arch=gfx950", "-fno-gpu-flush-denormals-to-zero",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
          "-Wno-unused-command-line-argument"]
SOURCES = {
    "quant.hip": ["-ffp-contract=off"],
    "attn_fwd.hip": [],
    "attn_short.hip": [],
    "api.cpp": ["-x", "hip"],
}


HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g"]


def _compile(name: str, extra, verbose: bool, objdir: str = OBJ) -> str:
    src = os.path.join(CSRC, name)
    obj = os.path.join(objdir, name + ".o")
    cmd = [HIPCC] + COMMON + extra + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {name}:\n{err}")
    if err.strip() and verbose:
        print(err)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda kv: _compile(kv[0], kv[1], verbose), SOURCES.items()))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_host_sanitized(path: str, verbose: bool = False) -> str:
    objdir = os.path.join(os.path.dirname(os.path.abspath(path)), "_asan_obj")
    os.makedirs(objdir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda kv: _compile(kv[0], kv[1] + HOST_SANITIZE, verbose, objdir),
                           SOURCES.items()))
    cmd = ([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + HOST_SANITIZE
           + ["-shared-libsan", "-o", path] + objs)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return path


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
