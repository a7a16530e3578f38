"""Builds a copy of libkpool.so whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer (the device
code is built as usual), plus the host-only ABI driver linked against it, under tests/sanitize/_build/.

    python tests/sanitize/build_sanitized.py

The sanitizers apply to host code only: each -fsanitize flag on a hipcc line is scoped with -Xarch_host.  Used by
tests/test_sanitize.py on the CPU; nothing here runs on a GPU."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
from sparse_attention_kpool_amd import build as B  # noqa: E402

OUT = os.path.join(HERE, "_build")
LIB = os.path.join(OUT, "libkpool_san.so")
DRIVER = os.path.join(OUT, "abi_driver")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libasan"]


def clang_rt_dir() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no clang AddressSanitizer runtime under /opt/rocm/llvm")
    return os.path.dirname(hits[-1])


def _compile(src: str) -> str:
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    cmd = [B.hipcc(), *B.COMPILE_FLAGS, *B.FILE_FLAGS.get(os.path.basename(src), []), *HOST_SAN, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}{r.stderr}")
    return obj


def build(jobs: int = 8) -> tuple:
    os.makedirs(OUT, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, B.sources()))
    subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *HOST_SAN, "-o", LIB, *objs],
                   check=True, capture_output=True)
    clang = "/opt/rocm/llvm/bin/clang"
    subprocess.run([clang, "-O1", "-g", "-fsanitize=address,undefined", "-shared-libasan", "-fno-omit-frame-pointer",
                    "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "abi_driver.c"), "-o", DRIVER,
                    "-L", OUT, "-lkpool_san", f"-Wl,-rpath,{OUT}", f"-Wl,-rpath,{clang_rt_dir()}"],
                   check=True, capture_output=True)
    return LIB, DRIVER


if __name__ == "__main__":
    print(build())
