"""Host-side sanitizer run of the C ABI's validation.

Builds every source of libbsa.so with its host pass under AddressSanitizer
and UndefinedBehaviorSanitizer (the gfx950 device code is built as usual)
into _build/asan/libbsa_asan.so, then runs tests/test_abi.py against that
library in a child process with the ASan runtime preloaded.  test_abi makes
no GPU call: every call it makes returns from host validation, so this runs
on a machine without a GPU.

    python -m dlm_bsa_block_amd.sanitize_check
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

from . import build as bb

OUT = os.path.join(os.path.dirname(bb.HERE), "_build", "asan")
LIB = os.path.join(OUT, "libbsa_asan.so")
# host pass only: each sanitizer flag goes behind -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def _llvm(tool: str) -> str:
    return os.path.join(os.path.dirname(os.path.realpath(bb._hipcc())), "..", "llvm", "bin", tool)


def _compile(src: str) -> str:
    obj = os.path.join(OUT, src.replace(".hip", ".o"))
    cmd = [bb._hipcc(), *[f for f in bb.FLAGS if f != "-O3"], "-O1", "-g", *HOST_SAN, "-c",
           os.path.join(bb.CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed for {src}:\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(bb.SOURCES))) as ex:
        objs = list(ex.map(_compile, bb.SOURCES))
    rocm = os.path.realpath(os.path.join(os.path.dirname(os.path.realpath(bb._hipcc())), ".."))
    # host link of the objects (each carries its own device code): the host compiler driver
    cmd = [_llvm("clang++"), "-shared", "-fsanitize=address,undefined", "-shared-libsan", "-o", LIB, *objs,
           "-L" + os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return LIB


def run() -> int:
    lib = build()
    rt = subprocess.run([_llvm("clang"), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    env = dict(os.environ, BSA_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    root = os.path.dirname(bb.HERE)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(root, "tests", "test_abi.py")], cwd=root, env=env)
    return r.returncode


if __name__ == "__main__":
    sys.exit(run())
