"""Build libfwmem.so in-tree for gfx950 with hipcc (cross-compiles without a GPU).

    python -m linear_attention_scan_amd.build [--jobs N] [--verbose]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfwmem.so")
SOURCES = ["fwmem_api.cpp", "fwmem_scan.hip", "fwmem_scan_split.hip", "fwmem_prep_split.hip", "fwmem_step.hip",
           "fwmem_segment.hip", "fwmem_znorm.hip", "fwmem_scan_pv.hip", "fwmem_scan_add.hip", "fwmem_backward.hip", "fwmem_backward_chunk.hip",
           "fwmem_noalloc.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay disabled (the compiler would otherwise form
    # v_pk_* fp32 ops from plain float code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs (no accumulator-register copies around VALU use)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(jobs: int = 3, verbose: bool = False) -> str:
    """Compile every source and link libfwmem.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libfwmem_asan.so")


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime of the ROCm clang that hipcc drives ("" if absent)."""
    r = subprocess.run([os.path.join(os.path.dirname(HIPCC), "..", "llvm", "bin", "clang"),
                        "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path):
        r = subprocess.run([os.path.join(os.path.dirname(HIPCC), "..", "llvm", "bin", "clang"),
                            "--print-resource-dir"], capture_output=True, text=True)
        path = os.path.join(r.stdout.strip(), "lib", "linux", "libclang_rt.asan-x86_64.so")
    return path if os.path.exists(path) else ""


def build_sanitized(verbose: bool = False) -> str:
    """A copy of the library whose host-side C-ABI layer (fwmem_api.cpp) is built with
    AddressSanitizer and UndefinedBehaviorSanitizer, for the CPU checks of the ABI. The
    sanitizer flags apply to the host compilation only (each -fsanitize= follows
    -Xarch_host); the kernels' objects are those of build(). Load it with the ASan runtime
    preloaded. Returns the library path."""
    objs = [os.path.join(BUILD, os.path.splitext(src)[0] + ".o") for src in SOURCES if src != "fwmem_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build(jobs=8, verbose=verbose)
    os.makedirs(ASAN_DIR, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    api = os.path.join(ASAN_DIR, "fwmem_api.o")
    cmd = [HIPCC] + FLAGS + ["-O1", "-g", "-fno-omit-frame-pointer"] + san + [
        "-c", os.path.join(CSRC, "fwmem_api.cpp"), "-o", api]
    for c in (cmd, [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + san[:4] +
              ["-Xarch_host", "-shared-libsan", "-o", ASAN_LIB, api] + objs):
        if verbose:
            print(" ".join(c), flush=True)
        r = subprocess.run(c, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitizer build failed:\n{r.stdout}\n{r.stderr}")
    return ASAN_LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=3)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--sanitized", action="store_true",
                    help="also build the host-sanitizer copy of the ABI layer (CPU checks)")
    a = ap.parse_args(argv)
    print(build(jobs=a.jobs, verbose=a.verbose))
    if a.sanitized:
        print(build_sanitized(verbose=a.verbose))


if __name__ == "__main__":
    main()
