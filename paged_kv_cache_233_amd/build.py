"""Builds libpkv.so (HIP kernels for gfx950 + host allocator + C ABI) in
place, next to this file. Run as ``python -m paged_kv_cache_233_amd.build``."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpkv.so")
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")

SOURCES = ["abi.cpp", "errors.cpp", "allocator.cpp", "scheduler.cpp", "sha256.cpp", "cache_ops.hip",
           "decode.hip", "prefill.hip"]
# The host-only part (no HIP runtime): built alone, with sanitizers, by
# build_host_sanitized().
HOST_SOURCES = ["errors.cpp", "allocator.cpp", "scheduler.cpp", "sha256.cpp"]
HOST_LIB = os.path.join(HERE, "libpkv_host_asan.so")
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]

# Packed-FP32 VALU instructions are kept out of all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The prefill kernel keeps its MFMA accumulators in ordinary VGPRs: its
# softmax rescales them with VALU code on a branch, and accumulators in
# AGPRs were copied back and forth around that branch on every tile.
FILE_FLAGS = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    """Compile every source and link libpkv.so; returns its path."""
    with tempfile.TemporaryDirectory(prefix="pkv_build_") as tmp:
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
                   "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
            if src.endswith(".hip"):
                cmd += ["-x", "hip"] + DEVICE_FLAGS + FILE_FLAGS.get(src, [])
            cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
            _run(cmd, verbose)
            objs.append(obj)
        tmp_lib = LIB + ".tmp"
        _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp_lib] + objs, verbose)
        os.replace(tmp_lib, LIB)
    return LIB


def build_host_sanitized(verbose: bool = False) -> str:
    """The host-only sources (allocator, scheduler, SHA-256, status
    plumbing) built with g++ and AddressSanitizer + UndefinedBehaviorSanitizer
    into libpkv_host_asan.so. A process that loads it needs the ASan runtime
    preloaded (LD_PRELOAD of g++'s libasan.so)."""
    with tempfile.TemporaryDirectory(prefix="pkv_host_asan_") as tmp:
        objs = []
        for src in HOST_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            _run(["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-Wall"] + SANITIZE +
                 ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, src),
                  "-o", obj], verbose)
            objs.append(obj)
        tmp_lib = HOST_LIB + ".tmp"
        _run(["g++", "-shared", "-fPIC"] + SANITIZE + ["-o", tmp_lib] + objs, verbose)
        os.replace(tmp_lib, HOST_LIB)
    return HOST_LIB


def asan_runtime() -> str:
    """Path of g++'s AddressSanitizer runtime (for LD_PRELOAD)."""
    return subprocess.run(["g++", "-print-file-name=libasan.so"], stdout=subprocess.PIPE,
                          text=True, check=True).stdout.strip()


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # The host pass of hipcc does not know the device-only feature flag; drop
    # that one line of noise and show everything else.
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("build step failed: " + " ".join(cmd))
    if out.strip() and verbose:
        print(out)


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
