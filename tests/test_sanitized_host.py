"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library is rebuilt with its host code instrumented (hipcc, every -fsanitize= behind -Xarch_host,
so the device code is compiled as usual and never instrumented), the oracle with clang's
-fsanitize=address,undefined, and the rest of the CPU suite runs against both builds in a child
process with the sanitizer runtime preloaded. That covers the multithreaded packers (pext loops over
raw pointers, shared sign words merged at range edges), descriptor checks, validation and unpacking
("Breaking the 1.58-bit Barrier for Ternary LLMs", Sec. II-A and Fig. 2: the packing they guard), the
launch-side argument checks, and the oracle. Any report aborts the child, and the test fails.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "bit_gemv_decode_amd", "csrc")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.sanitize
def test_cpu_suite_under_asan_and_ubsan(tmp_path):
    rt = _runtime()
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    from bit_gemv_decode_amd import build as B

    common = ["-O1", "-g", "-std=c++20", "-fPIC", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
              "-I", CSRC, *HOST_SAN]

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        lang = ["-x", "hip", f"--offload-arch={B.ARCH}", "-Xclang", "-target-feature", "-Xclang",
                "-packed-fp32-ops"] if src.endswith(".hip") else []
        r = subprocess.run(["hipcc", *common, *lang, "-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with ThreadPoolExecutor(8) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    lib = str(tmp_path / "libternary_gemv_san.so")
    r = subprocess.run(["hipcc", f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *HOST_SAN, "-o", lib, *objs,
                        "-lpthread"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    olib = str(tmp_path / "liboracle_san.so")
    r = subprocess.run(["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-shared", "-fPIC", "-std=c99",
                        "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-o", olib,
                        os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, LD_PRELOAD=rt, TG_LIB_PATH=lib, ORACLE_LIB=olib, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m",
                        "not gpu and not sanitize", os.path.join(ROOT, "tests")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert " passed" in r.stdout and "failed" not in r.stdout
