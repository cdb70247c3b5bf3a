"""Build libpp.so in-tree for gfx950 with hipcc.

Usage: python -m personaplex_temporal_transformer_amd.build   (or build() from Python).
Every call recompiles all sources (it is the "does it build" check as well)."""

import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libpp.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]
# Packed FP32 instructions are kept out of the device code.
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip"] + DEVICE + COMMON + ["-c", src, "-o", obj]
    else:
        cmd = [HIPCC] + DEVICE + COMMON + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (src, " ".join(cmd), msg))
    return obj, msg


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    for _, msg in results:
        if msg.strip() and verbose:
            print(msg, file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "--offload-arch=" + ARCH, "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stdout + r.stderr))
    os.replace(tmp, OUT)
    return OUT


# Host code under AddressSanitizer (device code as usual): libpp_asan.so next to libpp.so and
# the C++ driver tests/asan/abi_driver that calls every entry point through it.
ASAN_OUT = os.path.join(PKG, "libpp_asan.so")
ASAN_DIR = os.path.join(BUILD_DIR, "asan")
ASAN_DRIVER = os.path.join(ROOT, "tests", "asan", "abi_driver")
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile_asan(src):
    obj = os.path.join(ASAN_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + lang + DEVICE + COMMON + ASAN_FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (src, " ".join(cmd), r.stdout + r.stderr))
    return obj


def build_asan():
    os.makedirs(ASAN_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile_asan, srcs))
    steps = [
        [HIPCC, "-shared", "--offload-arch=" + ARCH] + ASAN_FLAGS + ["-o", ASAN_OUT] + objs,
        [HIPCC, "-O1", "-std=c++17", "-I", INCLUDE] + ASAN_FLAGS +
        [os.path.join(ROOT, "tests", "asan", "abi_driver.cpp"), "-L" + PKG, "-lpp_asan",
         "-Wl,-rpath,$ORIGIN/../../personaplex_temporal_transformer_amd", "-o", ASAN_DRIVER],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("asan build failed:\n%s\n%s" % (" ".join(cmd), r.stdout + r.stderr))
    return ASAN_OUT, ASAN_DRIVER


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_asan())
