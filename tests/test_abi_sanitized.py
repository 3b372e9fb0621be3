"""The C ABI's host code under AddressSanitizer and UBSan (CPU only).

The library's host side -- argument and shape checks, workspace layouts,
table construction, schedules, the loading controller -- is rebuilt with the
sanitizers on the host compilation (device code unchanged), loaded in a
fresh Python process with the ASan runtime preloaded, and the ABI and
controller tests run against it.  Any sanitizer report (out-of-bounds or
use-after-free access, undefined behaviour such as an out-of-range enum
load or a signed overflow) fails the run."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale(lib, src_dir, header):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = [os.path.join(src_dir, f) for f in os.listdir(src_dir)] + [header]
    return any(os.path.getmtime(f) > t for f in srcs)


def test_abi_tests_pass_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from rag_kv_cache_layer_amd import build_sanitized as bs
    from rag_kv_cache_layer_amd.build import CSRC, INCLUDE
    if _stale(bs.SAN_LIB, CSRC, os.path.join(INCLUDE, "cacheblend.h")):
        bs.build()
    env = dict(os.environ)
    env["LD_PRELOAD"] = bs.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["CB_LIB"] = bs.SAN_LIB
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_controller.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    out = r.stdout
    assert "runtime error" not in out and "Sanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
