"""Build libmoe_nvfp4.so in-tree with hipcc for gfx950.

Usage: ``python -m nvfp4_w4a4_mixture_amd.build`` (also called by
``__graft_entry__.build()``).  Every source is compiled on every call.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "lib")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libmoe_nvfp4.so"
SOURCES = ["quantize.hip", "route.hip", "ffn.hip", "combine.hip", "prune.hip", "shared.hip", "rotate.hip", "api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",  # every float step of the quantizer is one IEEE operation
    # packed FP32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Host-code sanitizers for a checking build (AddressSanitizer + UndefinedBehaviorSanitizer).  Each
# flag is applied to the host compilation only; device code is built exactly as in the product.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZE_DIR = os.path.join(BUILD_DIR, "sanitize")


def _compile(src: str, build_dir: str = BUILD_DIR, defines=(), extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *extra, *[f"-D{d}" for d in defines], *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out_dir: str = OUT_DIR, build_dir: str = BUILD_DIR, defines=(),
          sanitize: bool = False) -> str:
    """Compile every source and link ``<out_dir>/libmoe_nvfp4.so``; returns its path.

    ``defines`` (NAME=VALUE strings) override compile-time tile parameters.  ``sanitize``
    instruments the host code with AddressSanitizer and UndefinedBehaviorSanitizer (the library
    then needs the ASan runtime preloaded); by default it goes to ``_build/sanitize/``."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    if sanitize and out_dir == OUT_DIR:
        out_dir = build_dir = SANITIZE_DIR
    extra = SANITIZE_HOST if sanitize else []
    os.makedirs(build_dir, exist_ok=True)
    os.makedirs(out_dir, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, defines, extra), SOURCES))
    tmp = os.path.join(out_dir, LIB_NAME + ".tmp")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    out = os.path.join(out_dir, LIB_NAME)
    shutil.move(tmp, out)
    if verbose:
        print("built", out)
    return out


def asan_runtime() -> str:
    """Path of the ASan runtime matching hipcc (preloaded to run a sanitized build)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"ASan runtime not found (hipcc said {path!r})")
    return path


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
