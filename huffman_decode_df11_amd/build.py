"""Build libdf11.so in-tree: HIP kernels for gfx950 with hipcc, host C++ with g++.

    python -m huffman_decode_df11_amd.build

The library lands in huffman_decode_df11_amd/_build/libdf11.so, next to
df11_c_api_check, a host program that uses the C ABI alone (no Python), and
df11_segment_bounds_check, a host program that checks the decode kernels'
per-segment address arithmetic (segment_plan.h) on random and corrupt
segment records.

    python -m huffman_decode_df11_amd.build --sanitize

builds the same library with AddressSanitizer and UndefinedBehaviorSanitizer
in its host code (clang, the GPU code unchanged) into _build_san/, and the
oracle likewise; the CPU tests run against them with

    DF11_LIBRARY=huffman_decode_df11_amd/_build_san/libdf11.so \
    DF11_ORACLE_LIBRARY=oracle/_build_san/liborc.so \
    LD_PRELOAD=$(python -m huffman_decode_df11_amd.build --print-asan-runtime) \
    ASAN_OPTIONS=detect_leaks=0 python -m pytest tests -m "not gpu"
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(OUT_DIR, "libdf11.so")
C_API_CHECK = os.path.join(OUT_DIR, "df11_c_api_check")
BOUNDS_CHECK = os.path.join(OUT_DIR, "df11_segment_bounds_check")
SAN_DIR = os.path.join(PKG, "_build_san")
LLVM_BIN = "/opt/rocm/llvm/bin"
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_SOURCES = ["decode.hip", "decode_gemm.hip", "encode.hip"]
CPP_SOURCES = ["host_codebook.cpp", "host_encode.cpp", "host_validate.cpp"]

# Packed FP32 instructions are kept out of every HIP object.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]
CXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]


def _run_all(cmds):
    procs = [(c, subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)) for c in cmds]
    failed = []
    for c, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            failed.append((c, text))
        elif text.strip():
            sys.stderr.write(text)
    if failed:
        msg = "\n\n".join(" ".join(c) + "\n" + t for c, t in failed)
        raise RuntimeError("libdf11 build failed:\n" + msg)


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    cmds, objs = [], []
    for src in HIP_SOURCES:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(OUT_DIR, src + ".o")
        cmds.append([HIPCC, *HIP_FLAGS, "-c", path, "-o", obj])
        objs.append(obj)
    for src in CPP_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        cmds.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    if verbose:
        for c in cmds:
            print(" ".join(c))
    _run_all(cmds)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run_all([[HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp, *objs]])
    os.replace(tmp, LIB)
    # the C ABI example/check program, linked against the library beside it
    tmp = C_API_CHECK + ".tmp%d" % os.getpid()
    _run_all([[HIPCC, "-O2", "-std=c++17", "--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "-I", INCLUDE, os.path.join(CSRC, "examples", "c_api_check.cpp"),
               "-L", OUT_DIR, "-ldf11", "-Wl,-rpath,$ORIGIN", "-o", tmp]])
    os.replace(tmp, C_API_CHECK)
    tmp = BOUNDS_CHECK + ".tmp%d" % os.getpid()
    _run_all([["g++", "-O2", "-std=c++17", "-Wall", os.path.join(CSRC, "checks", "segment_bounds_check.cpp"),
               "-o", tmp]])
    os.replace(tmp, BOUNDS_CHECK)
    return LIB


SAN_FLAGS = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime of the clang that builds the
    sanitized library (to preload into an interpreter that loads it)."""
    out = subprocess.run([os.path.join(LLVM_BIN, "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True).stdout.strip()
    return out


def build_sanitized(verbose: bool = False) -> str:
    """libdf11.so with host-side AddressSanitizer + UndefinedBehaviorSanitizer
    in _build_san/: HIP sources through hipcc with every -fsanitize= behind
    -Xarch_host (device code is built as usual), host C++ through clang++.
    The shared sanitizer runtime is linked, so that a Python process can
    load the library with the runtime preloaded."""
    os.makedirs(SAN_DIR, exist_ok=True)
    host_san = []
    for f in SAN_FLAGS:
        host_san += ["-Xarch_host", f]
    cmds, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(SAN_DIR, src + ".o")
        cmds.append([HIPCC, *HIP_FLAGS, *host_san, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CPP_SOURCES:
        obj = os.path.join(SAN_DIR, src + ".o")
        cmds.append([os.path.join(LLVM_BIN, "clang++"), *CXX_FLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, src),
                     "-o", obj])
        objs.append(obj)
    if verbose:
        for c in cmds:
            print(" ".join(c))
    _run_all(cmds)
    lib = os.path.join(SAN_DIR, "libdf11.so")
    _run_all([[HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-shared-libsan", "-Xarch_host",
               "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", lib, *objs]])
    return lib


if __name__ == "__main__":
    if "--print-asan-runtime" in sys.argv:
        print(asan_runtime())
    elif "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
        from oracle import oracle
        print(oracle.build_sanitized())
    else:
        print(build(verbose="-v" in sys.argv))
