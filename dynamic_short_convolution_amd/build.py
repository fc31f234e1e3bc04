"""Builds libdynconv.so (HIP kernels + C ABI) for gfx950 with hipcc, in the package dir.

Usage: python -m dynamic_short_convolution_amd.build   (or build() from Python).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libdynconv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = [
    "dynconv_abi.hip",
    "dynconv_stream.hip",
    "dynconv_stream_f32.hip",
    "dynconv_stream_bf16.hip",
    "dynconv_stream_f16.hip",
    "dynconv_lowrank.hip",
    "dynconv_lowrank_f32.hip",
    "dynconv_lowrank_bf16.hip",
    "dynconv_lowrank_f16.hip",
    "dynconv_lowrank_fast.hip",
    "dynconv_decode.hip",
    "dynconv_gemm.hip",
]

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 are generated from ordinary float code.
COMPILE_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang",
    "-target-feature",
    "-Xclang",
    "-packed-fp32-ops",
    # matrix-core results in ordinary VGPRs: no v_accvgpr_read copies before they are used
    "-mllvm",
    "-amdgpu-mfma-vgpr-form",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMPILE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compiles every source and links libdynconv.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


# Host-side code only, with AddressSanitizer and UndefinedBehaviorSanitizer on the host
# compile. Each object embeds the same device bundle of an empty source file instead of its
# kernels, so the library registers no kernels: only argument checking, planning and size
# queries can run (a launch would fail). Loaded with the clang ASan runtime
# preloaded (SANITIZER_RUNTIME) by a process that selects it through DYNCONV_LIBRARY.
ASAN_DIR = os.path.join(PKG_DIR, "_build_asan")
ASAN_LIB_PATH = os.path.join(ASAN_DIR, "libdynconv_hostsan.so")
SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]


def sanitizer_runtime() -> str:
    """Path of the clang ASan runtime matching hipcc's compiler."""
    res = subprocess.run([os.path.join(os.path.dirname(HIPCC), "..", "lib", "llvm", "bin", "clang"),
                          "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"no ASan runtime found ({res.stdout} {res.stderr})")
    return path


def build_host_sanitized() -> str:
    """Builds the host-only sanitized library; returns its path."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    empty_src = os.path.join(ASAN_DIR, "empty.hip")
    empty_bin = os.path.join(ASAN_DIR, "empty.fatbin")
    with open(empty_src, "w") as f:
        f.write("// no kernels\n")
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "--cuda-device-only", "--no-offload-new-driver", "-c",
           empty_src, "-o", empty_bin]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"empty device bundle failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")

    def one(src: str) -> str:
        obj = os.path.join(ASAN_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, "-x", "hip", "--cuda-host-only", "--no-offload-new-driver", "-Xclang", "-fcuda-include-gpubinary",
               "-Xclang", empty_bin, "-O1", "-g", "-std=c++17", "-fPIC", *SANITIZE_FLAGS, "-c",
               os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, SOURCES))
    cmd = [HIPCC, "-shared", "-fPIC", *SANITIZE_FLAGS, "-shared-libasan", *objs, "-o", ASAN_LIB_PATH]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return ASAN_LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
