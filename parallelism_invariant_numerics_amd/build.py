"""Build libiso.so (HIP kernels for gfx950 + the C-ABI host code) in-tree.

    python parallelism_invariant_numerics_amd/build.py

hipcc cross-compiles for gfx950 without a GPU.  Device code is built with
FP contraction off and without fast-math, so every kernel that shares a
device function rounds it the same way, and with packed-FP32 instruction
selection disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libiso.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

DEVICE_SOURCES = ["gemm.hip", "gemm_rows.hip", "lmhead.hip", "moe.hip", "norm.hip", "cpr.hip"]
HOST_SOURCES = ["iso_host.cpp", "sha256.cpp", "identity.cpp"]

COMMON = ["-O3", "-fPIC", "-std=c++20", "-Wall", "-I", os.path.join(ROOT, "include")]
DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-ffp-contract=off", "-fno-fast-math",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device feature flag: drop that notice
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for s in DEVICE_SOURCES:
        o = os.path.join(OBJ, s.replace(".hip", ".o"))
        jobs.append([HIPCC, *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
    for s in HOST_SOURCES:
        o = os.path.join(OBJ, s.replace(".cpp", ".o"))
        jobs.append([HIPCC, *COMMON, "-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for f in [ex.submit(_run, j) for j in jobs]:
            f.result()
    objs = [j[-1] for j in jobs]
    tmp = LIB + f".tmp{os.getpid()}"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def device_asm(source: str, out_path: str) -> str:
    """The gfx950 assembly of one device source, with the library's flags."""
    _run([HIPCC, *COMMON, *DEVICE_FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, source),
          "-o", out_path])
    return out_path


# CPU build of the host code under AddressSanitizer and UndefinedBehavior-
# Sanitizer: the C ABI's checks, the identities and SHA-256, with the kernel
# launchers replaced by stubs that launch nothing (host_stubs.cpp).  g++ on
# host sources only; no GPU code is built with a sanitizer.
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer", "-g", "-O1"]


def build_host_sanitized(out_path: str) -> str:
    srcs = [os.path.join(CSRC, f) for f in HOST_SOURCES + ["host_stubs.cpp"]]
    _run(["g++", "-std=c++17", "-fPIC", "-shared", "-Wall", *SANITIZE, "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", *srcs,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", out_path])
    return out_path


if __name__ == "__main__":
    build(verbose=True)
