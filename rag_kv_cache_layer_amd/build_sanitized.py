"""Host-sanitized build of the fusor library (AddressSanitizer + UBSan on the
host code only; the gfx950 device code is built as usual).

The host side of the C ABI -- argument and shape checks, workspace layout,
launch sequencing -- is compiled with -fsanitize=address,undefined (UBSan
errors abort) into _build/san/libcacheblend_san.so.  tests/test_abi_sanitized.py
loads it (CB_LIB) under the ASan runtime and runs the ABI tests, which
exercise every error path without touching a GPU.  Device code is never
sanitized.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

from .build import CSRC, FLAGS, HIPCC, ROOT, SOURCES

SAN_DIR = os.path.join(ROOT, "_build", "san")
SAN_LIB = os.path.join(SAN_DIR, "libcacheblend_san.so")
# every sanitizer flag applies to the host compilation only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to LD_PRELOAD into python)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                       stderr=subprocess.DEVNULL, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the ASan runtime of the HIP compiler was not found")
    return path


def build(jobs: int = 8) -> str:
    os.makedirs(SAN_DIR, exist_ok=True)
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SAN
    objs = [os.path.join(SAN_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]

    def one(so):
        s, o = so
        r = subprocess.run([HIPCC, *flags, "-c", os.path.join(CSRC, s), "-o", o], stdout=subprocess.PIPE,
                           stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized build of {s} failed:\n{r.stdout}")
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(one, zip(SOURCES, objs)))
    tmp = SAN_LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN, "-shared-libsan", "-o", tmp,
                        *objs], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitized link failed:\n" + r.stdout)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    print(build())
