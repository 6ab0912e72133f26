"""The host-side argument checks of libkvx under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is built again with both sanitizers on its host code only (the GPU code is built as
usual and is never instrumented) into a temporary directory, and the host-only ABI tests
(test_abi_host.py: every validation error path, workspace queries, the budget) run against it
in a child process with the sanitizer runtime preloaded.  An invalid memory access or undefined
behaviour (signed overflow in a size computation, a shift out of range, a misaligned access)
in the checks aborts the child and fails this test.  No GPU is needed: every call under test
fails validation before any device work.
"""
import glob
import os
import subprocess
import sys

import pytest

from cross_model_kv_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# sanitizer options for the host pass only; each one follows -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _runtime():
    llvm = os.path.join(os.path.dirname(os.path.realpath(build.HIPCC)), "..", "llvm")
    hits = sorted(glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def _build(out_dir):
    flags = [f for f in build.FLAGS if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer"] + HOST_SAN
    procs, objs = [], []
    for src in build.SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([build.HIPCC, *flags, "-c", os.path.join(build.CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p, src in zip(procs, build.SOURCES):
        _, err = p.communicate()
        assert p.returncode == 0, f"hipcc failed on {src}:\n{err[-3000:]}"
    lib = os.path.join(out_dir, "libkvx_san.so")
    r = subprocess.run([build.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, *HOST_SAN, "-shared-libsan",
                        "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return lib


CHILD = """
import sys
from cross_model_kv_amd import kvx
kvx.LIB_PATH = sys.argv[1]
import pytest
sys.exit(pytest.main([sys.argv[2], "-q", "-p", "no:cacheprovider", "-m", "not gpu"]))
"""


def test_host_checks_clean_under_sanitizers(tmp_path):
    rt = _runtime()
    if rt is None or not os.path.exists(build.HIPCC):
        pytest.skip("no hipcc or no clang sanitizer runtime in this image")
    lib = _build(str(tmp_path))
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-c", CHILD, lib, os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]
