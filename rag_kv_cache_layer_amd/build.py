"""Build of the gfx950 fusor library (libcacheblend.so), in-tree.

Every HIP source under ``csrc/`` is compiled with ``hipcc --offload-arch=gfx950``
into an object under ``_build/`` and linked into
``rag_kv_cache_layer_amd/libcacheblend.so``.  Packed fp32 instructions are
switched off for device code (``-target-feature -packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcacheblend.so")
SOURCES = ("rope.hip", "norm.hip", "select.hip", "gemm.hip", "attn.hip", "fp8.hip", "kv8.hip", "copy.hip", "analytics.hip", "api.hip")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [l for l in r.stdout.splitlines() if "not a recognized feature" not in l]
    return r.returncode, "\n".join(lines)


def build(verbose: bool = False, jobs: int = 8, out: str = LIB, defines=(), build_dir: str = BUILD) -> str:
    """Compile every source and link the shared library; returns its path.
    defines: extra -D macros (kernel tuning knobs); out / build_dir: where the
    objects and the library go."""
    os.makedirs(build_dir, exist_ok=True)
    objs = [os.path.join(build_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, *["-D" + d for d in defines], "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(cmds))) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, log) in zip(cmds, results):
        if verbose and log.strip():
            print(log, file=sys.stderr)
        if rc != 0:
            raise RuntimeError("hipcc failed: " + " ".join(cmd) + "\n" + log)
    tmp = out + ".tmp"
    rc, log = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        raise RuntimeError("link failed\n" + log)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
