"""Build libmoe_w4a16.so (HIP, gfx950) and libmoe_pool_host.so (host-only
slot-pool build with a memcpy backend, used by CPU tests) in-tree.

    python -m int4_weight_only_router_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INC = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_w4a16.so")
POOL_HOST_LIB = os.path.join(PKG, "libmoe_pool_host.so")

HIP_SOURCES = ["moe_api.cpp", "k_route.hip", "k_permute.hip", "k_ffn_decode.hip", "k_shared_gemv.hip",
               "k_ffn_grouped.hip", "k_ffn_small.hip", "k_combine.hip", "k_combine_route.hip", "k_quant.hip", "pool_hip.cpp",
               "prepack_host.cpp"]
HEADERS = ["moe_common.h", "k_w4_frag.h", "k_decode_frag.h", "k_sort_common.h", "k_combine_tile.h",
           "pool_core.h", "trace.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM_LIB = "/opt/rocm/lib"
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
    # no packed-fp32 instructions are generated (scalar fp32 only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-result",
    "-I", INC, "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n%s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if err.strip():
        sys.stderr.write(err + "\n")


def _deps_mtime():
    files = [os.path.join(CSRC, f) for f in HIP_SOURCES + HEADERS + ["pool_fake.cpp"]]
    files.append(os.path.join(INC, "moe_w4a16.h"))
    return max(os.path.getmtime(f) for f in files)


def up_to_date() -> bool:
    return all(os.path.exists(p) and os.path.getmtime(p) >= _deps_mtime()
               for p in (LIB, POOL_HOST_LIB))


def build(force: bool = True, jobs: int = 8) -> str:
    if not force and up_to_date():
        return LIB
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        _run([HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, HIP_SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    # roctx ranges (trace.h) come from the ROCm profiler SDK's roctx library
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs +
         ["-L", ROCM_LIB, "-Wl,-rpath," + ROCM_LIB, "-lrocprofiler-sdk-roctx"])
    os.replace(tmp, LIB)
    tmp = POOL_HOST_LIB + ".tmp%d" % os.getpid()
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", "-D__HIP_PLATFORM_AMD__",
          "-I", INC, "-I", CSRC, "-I", "/opt/rocm/include",
          os.path.join(CSRC, "pool_fake.cpp"), "-o", tmp])
    os.replace(tmp, POOL_HOST_LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True))
