"""Build libsgemm_f32.so in-tree with hipcc for gfx950.

    python -m fp32_gemm_08_amd.build

Each source is compiled to an object (in parallel) under ``_build/`` and linked
into ``fp32_gemm_08_amd/libsgemm_f32.so``.  Packed FP32 instructions are kept
out of the device code (``-packed-fp32-ops``); no fast-math flags are used.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsgemm_f32.so")

SOURCES = ["sgemm_api.cpp", "k_naive.hip", "k_tiled.hip", "k_regblock.hip", "k_mfma.hip", "k_mfma_lp.hip", "k_lp16.hip", "k_splitk.hip",
           "k_transpose.hip", "k_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsgemm_f32.so)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function"]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags() + list(extra) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


# Debug variants, built next to the library on request and loaded through
# SGEMM_F32_LIBRARY (the product build is libsgemm_f32.so):
#   poison    every LDS stage NaN-filled before it is staged (SGEMM_DEBUG_POISON_LDS)
#   sanitize  host code under AddressSanitizer and UndefinedBehaviorSanitizer
#             (device code as in the library), for the argument checks,
#             planning and entry points of the C ABI on a machine without a
#             GPU; load it with the sanitizer runtime preloaded
#             (sanitizer_runtime())
VARIANTS = {
    "poison": ["-DSGEMM_DEBUG_POISON_LDS"],
    "sanitize": ["-DSGEMM_DEBUG_SANITIZE", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-shared-libsan"],
}


def variant_path(variant: str) -> str:
    return os.path.join(PKG, f"libsgemm_f32_{variant}.so")


def sanitizer_runtime() -> str:
    """Path of the clang AddressSanitizer runtime the sanitize variant links."""
    r = subprocess.run([hipcc(), "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return path


def build(verbose: bool = False, extra=(), variant: str = "") -> str:
    if variant and variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    if variant:
        global BUILD
        saved, BUILD = BUILD, os.path.join(BUILD, variant)
        try:
            return _build(verbose, list(extra) + VARIANTS[variant], variant_path(variant), variant)
        finally:
            BUILD = saved
    return _build(verbose, extra, LIB, "")


def _build(verbose, extra, lib, variant) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-shared-libsan"] if variant == "sanitize" else []
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + link_extra + ["-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    args = sys.argv[1:]
    var = ""
    if args and args[0].startswith("--variant="):
        var = args.pop(0).split("=", 1)[1]
    build(verbose=True, extra=args, variant=var)
