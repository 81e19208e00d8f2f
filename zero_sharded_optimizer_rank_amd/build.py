"""Build libzero_shard.so for gfx950 in-tree with hipcc.

Floating-point flags matter for results: no contraction into FMA, correctly
rounded fp32 division and square root, denormals kept, and no packed fp32
instructions.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libzero_shard.so")
CALIB_LIB = os.path.join(HERE, "libzero_calib.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FP_FLAGS = [
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
]
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    kobj = os.path.join(BUILD_DIR, "zero_kernels.o")
    uobj = os.path.join(BUILD_DIR, "zero_units.o")
    nobj = os.path.join(BUILD_DIR, "zero_noalloc.o")
    hobj = os.path.join(BUILD_DIR, "zero_host.o")
    oobj = os.path.join(BUILD_DIR, "zero_offload.o")
    _run([HIPCC, "-x", "hip", *COMMON, *FP_FLAGS, *DEVICE_FLAGS, "-c",
          os.path.join(CSRC, "zero_kernels.hip"), "-o", kobj])
    _run([HIPCC, "-x", "hip", *COMMON, *FP_FLAGS, *DEVICE_FLAGS, "-c",
          os.path.join(CSRC, "zero_units.hip"), "-o", uobj])
    _run([HIPCC, "-x", "hip", *COMMON, *FP_FLAGS, *DEVICE_FLAGS, "-c",
          os.path.join(CSRC, "zero_noalloc.hip"), "-o", nobj])
    _run([HIPCC, *COMMON, "-ffp-contract=off", "-c", os.path.join(CSRC, "zero_host.cpp"),
          "-o", hobj])
    # host Adam of the offload form: IEEE fp32, no contraction, errno-free sqrt
    _run([HIPCC, *COMMON, "-ffp-contract=off", "-fno-math-errno", "-pthread", "-c",
          os.path.join(CSRC, "zero_offload.cpp"), "-o", oobj])
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", kobj, uobj, nobj, hobj, oobj,
          "-o", tmp])
    os.replace(tmp, LIB)
    # measurement-only copy kernel, in a library of its own
    tmp = CALIB_LIB + ".tmp"
    _run([HIPCC, "-x", "hip", *COMMON, *DEVICE_FLAGS, "-shared",
          os.path.join(CSRC, "calib.hip"), "-o", tmp])
    os.replace(tmp, CALIB_LIB)
    build_c_example()
    return LIB


# A plain C program that runs the step through the C ABI with its own
# hipMalloc buffers (tests/c_abi_step.c, used by tests/test_gpu_c_abi.py).
C_EXAMPLE = os.path.join(BUILD_DIR, "c_abi_step")


def build_c_example() -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = C_EXAMPLE + ".tmp"
    _run(["gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
          "-I", INCLUDE, os.path.join(ROOT, "tests", "c_abi_step.c"), "-L", HERE, "-lzero_shard",
          "-L/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{HERE}", "-Wl,-rpath,/opt/rocm/lib",
          "-o", tmp])
    os.replace(tmp, C_EXAMPLE)
    return C_EXAMPLE


# Sanitizer builds of the host code, for CPU runs only: the C-ABI host
# sources built by g++ with AddressSanitizer + UndefinedBehaviorSanitizer
# ("asan") or ThreadSanitizer ("tsan"), linked with the unsanitized kernel
# objects of build() and with tests/host_sanitize_driver.cpp; "asan" also
# gives a library that the CPU tests load through ZERO_SHARD_LIB (with the
# ASan runtime preloaded).  The device code is never built with a sanitizer.
SAN_FLAGS = {
    "asan": ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer"],
    "tsan": ["-fsanitize=thread"],
}


def build_host_sanitized(kind: str) -> dict:
    flags = SAN_FLAGS[kind]
    out = os.path.join(BUILD_DIR, f"san_{kind}")
    os.makedirs(out, exist_ok=True)
    gxx = ["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-pthread", "-ffp-contract=off",
           "-fno-math-errno", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", INCLUDE,
           "-I", CSRC, *flags]
    objs = []
    for src in ("zero_host.cpp", "zero_offload.cpp"):
        o = os.path.join(out, src.replace(".cpp", ".o"))
        _run([*gxx, "-c", os.path.join(CSRC, src), "-o", o])
        objs.append(o)
    kobjs = [os.path.join(BUILD_DIR, f) for f in ("zero_kernels.o", "zero_units.o",
                                                  "zero_noalloc.o")]
    if not all(os.path.exists(k) for k in kobjs):
        build()
    link = ["-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64"]
    driver = os.path.join(out, "host_sanitize_driver")
    _run([*gxx, os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"), *objs, *kobjs, *link,
          "-o", driver])
    res = {"driver": driver}
    if kind == "asan":
        lib = os.path.join(out, "libzero_shard_asan.so")
        _run([*gxx, "-shared", *objs, *kobjs, *link, "-o", lib])
        res["lib"] = lib
    return res


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] in SAN_FLAGS:
        print(build_host_sanitized(sys.argv[1]))
    else:
        build()
    sys.exit(0)
