"""Build libbitkv.so for gfx950 with hipcc (in-tree, no JIT cache).

Each .hip file is compiled to an object in parallel, then linked into
``bit_kv_attention_amd/libbitkv.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbitkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["bitkv_api.hip", "pack.hip", "decode_approx.hip", "decode_approx.hip:q8", "decode_approx.hip:mx",
           "decode_approx.hip:fp4", "topk.hip", "correct.hip", "hybrid_layers.hip", "host_correct.cpp"]
# "file:variant" builds the file again into its own object with extra defines
VARIANT_DEFINES = {"q8": ["-DBKV_QUERY_INT8=1"], "mx": ["-DBKV_KEY_MXFP4=1"], "fp4": ["-DBKV_KEY_FP4=1"]}
# host-only source (the host-side exact correction), OpenMP over host threads
CXX = os.environ.get("CXX", "g++")
CXXFLAGS = ["-O3", "-fPIC", "-std=c++17", "-fopenmp", "-I", os.path.join(ROOT, "include")]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # packed fp32 VALU ops stay off (hipcc -O3 would otherwise form them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the codec needs IEEE fp32: keep denormals, correctly rounded divide
    "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
]


# The approximate scan only ever sees finite values and -inf: without IEEE
# mode min/max need no NaN quieting, so cross-lane maxima fold into one
# instruction.  The codec (pack.hip) keeps IEEE semantics.
EXTRA = {"decode_approx.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"]}


# The sanitizer build (CPU checks only): the host side of every source under
# clang's AddressSanitizer and UndefinedBehaviorSanitizer, linked into
# libbitkv_san.so, which the binding loads when BKV_SANITIZE=1 (run with the
# sanitizer runtime preloaded; see the oracle's own sanitizer build).  Device
# code is built as usual.
SAN_LIB = os.path.join(HERE, "libbitkv_san.so")
SAN_BUILD = os.path.join(HERE, "_build_san")
CLANGXX = os.environ.get("CLANGXX", "/opt/rocm/llvm/bin/clang++")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libsan"]
SAN_CXXFLAGS = ["-O1", "-g", "-fPIC", "-std=c++17", "-fopenmp=libgomp", "-fsanitize=address",
                "-fsanitize=undefined", "-fno-omit-frame-pointer", "-shared-libsan",
                "-I", os.path.join(ROOT, "include")]


def _compile(entry: str, sanitize: bool = False) -> str:
    src, _, variant = entry.partition(":")
    obj = os.path.join(SAN_BUILD if sanitize else BUILD,
                       os.path.splitext(src)[0] + (f"_{variant}" if variant else "") + ".o")
    if src.endswith(".cpp"):
        cmd = ([CLANGXX, *SAN_CXXFLAGS] if sanitize else [CXX, *CXXFLAGS]) + ["-c", os.path.join(CSRC, src),
                                                                         "-o", obj]
    else:
        cmd = [HIPCC, *FLAGS, *(SAN_HOST if sanitize else []), *EXTRA.get(src, []),
               *VARIANT_DEFINES.get(variant, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"compile failed on {entry}")
    return obj


# The read-ceiling probe bench.py --read-ceiling loads (measurement only; a
# library of its own, not part of libbitkv.so).
PROBE_SRC = os.path.join(HERE, "probe", "read_ceiling.hip")
PROBE_LIB = os.path.join(HERE, "libbkvprobe.so")


def build_probe(verbose: bool = False) -> str:
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-shared", PROBE_SRC, "-o", tmp]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES) + 1, os.cpu_count() or 4)) as ex:
        probe = ex.submit(build_probe, verbose)
        objs = list(ex.map(_compile, SOURCES))
        probe.result()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-lgomp", "-o", tmp]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    os.makedirs(SAN_BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda e: _compile(e, True), SOURCES))
    tmp = SAN_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_HOST, *objs, "-lgomp", "-o", tmp]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    print(build_sanitized(verbose=True) if "--sanitize" in sys.argv[1:] else build(verbose=True))
