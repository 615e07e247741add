"""Host-sanitized build of the library, for checking the C ABI's argument validation on
the CPU: AddressSanitizer and UndefinedBehaviorSanitizer instrument the host code
(validation, workspace carving, launch set-up); the gfx950 device code is compiled as
usual. The result, _build/san/libfourtune_san.so, is test infrastructure: the product
loads libfourtune.so only. It runs inside a process started with the ASan runtime
preloaded (tests/test_abi_sanitized_cpu.py).

    python -m bit_quantized_lora_fp4_amd.build_sanitize
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

from . import build as _b

SAN_DIR = os.path.join(_b.BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libfourtune_san.so")
SAN = ["-fno-gpu-sanitize -fsanitize=address,undefined -fno-sanitize-recover=undefined -fno-omit-frame-pointer -g"]


def asan_runtime() -> str:
    """The ASan runtime that matches the compiler (to preload into the test process)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def _compile(src):
    obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
    cmd = " ".join([_b.HIPCC, *_b.CFLAGS, *SAN, "-c", src, "-o", obj])
    r = subprocess.run(cmd, shell=True, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {cmd}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(SAN_DIR, exist_ok=True)
    srcs = _b.sources()
    with cf.ThreadPoolExecutor(min(len(srcs), 8)) as ex:
        objs = list(ex.map(_compile, srcs))
    cmd = " ".join([_b.HIPCC, f"--offload-arch={_b.ARCH}", "-shared", "-fPIC", *SAN, "-shared-libsan", *objs,
                    "-o", SAN_LIB])
    r = subprocess.run(cmd, shell=True, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {cmd}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


if __name__ == "__main__":
    build(verbose=True)
