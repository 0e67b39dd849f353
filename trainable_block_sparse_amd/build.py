"""Builds libinfv2.so (all HIP sources, gfx950 only) in the package directory.

    python -m trainable_block_sparse_amd.build [-v]
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libinfv2.so")
SOURCES = ["api.hip", "compress.hip", "scores.hip", "topk.hip", "attn.hip", "attn_bwd.hip"]

# Packed-fp32 instructions are disabled for all device code; the host pass
# reports the feature as unknown, which is harmless.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


HEADER = os.path.join(os.path.dirname(PKG), "include", "infv2.h")


def source_hash() -> str:
    """SHA-256 (16 hex digits) of every library source: csrc/ and the C
    header.  Compiled into the library (infv2_build_id) so that a run can show
    which sources the loaded library was built from."""
    h = hashlib.sha256()
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))] + [HEADER]
    for path in files:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str, verbose: bool, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if verbose and any(ln.strip() for ln in noise):
        print("\n".join(noise), file=sys.stderr)
    return obj


def _build(lib_path: str, build_dir: str, extra_compile, extra_link, verbose: bool) -> str:
    os.makedirs(build_dir, exist_ok=True)
    extra = [f'-DINFV2_SOURCE_HASH="{source_hash()}"', *extra_compile]
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *extra_link, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


def build(verbose: bool = False) -> str:
    """Compile every source and link libinfv2.so; returns the library path."""
    return _build(LIB, BUILD, (), (), verbose)


ASAN_LIB = os.path.join(PKG, "_build_asan", "libinfv2_asan.so")


def build_asan(verbose: bool = False) -> str:
    """The same library with AddressSanitizer on the host code only (the
    device code is built as usual), for CPU tests of the argument checks:
    _build_asan/libinfv2_asan.so.  A process that loads it must preload the
    ASan runtime (asan_runtime())."""
    flags = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    return _build(ASAN_LIB, os.path.dirname(ASAN_LIB), flags, ["-fsanitize=address", "-shared-libasan"],
                  verbose)


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    return r.stdout.strip()


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
