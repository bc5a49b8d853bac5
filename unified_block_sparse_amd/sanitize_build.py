"""Host-sanitizer build of libubs.so, for the CPU-side ABI tests.

    python -m unified_block_sparse_amd.sanitize_build

Compiles csrc/*.hip with AddressSanitizer and UndefinedBehaviorSanitizer on the HOST
side only (each flag behind -Xarch_host; device code is built as usual and never runs
in these tests) into unified_block_sparse_amd/_build_san/libubs_san.so. The argument
validation, workspace sizing and error reporting of the C ABI then run under both
sanitizers when the library is loaded with the AddressSanitizer runtime preloaded
(see asan_runtime()).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

from .build import ARCH, CSRC, HIPCC, INCLUDE, sources

HERE = os.path.dirname(os.path.abspath(__file__))
OUT_DIR = os.path.join(HERE, "_build_san")
OUT = os.path.join(OUT_DIR, "libubs_san.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
FLAGS = [f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=fast",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", f"-I{INCLUDE}", "-w", *HOST_SAN]


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (to be preloaded)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"AddressSanitizer runtime not found ({path!r})")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    r = subprocess.run([HIPCC, *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *HOST_SAN, "-shared-libasan",
                        *objs, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
    print(asan_runtime(), file=sys.stderr)
