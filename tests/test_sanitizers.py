"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The block ledger (block_pool.cpp: filled counts, reference counts, copy-on-write batches,
quarantines, host swap blocks, admission), the host half of the C ABI (abi.cpp: argument
checks, kernel selection, workspace layout) and the C oracle (pa_oracle.c) are rebuilt with
gcc's -fsanitize=address,undefined; the device half of the library is replaced by
tests/sanitize_stubs.cpp.  tests/sanitize_run.py then runs the ledger pins, the C++ ledger
against the oracle ledger on every workload script and on random scripts, the argument
checks of every entry point, decode planning on every workload shape and every oracle pin,
in a process with the sanitizer runtime preloaded.  Any report fails the test.

The bookkeeping checked here is that of "vLLM and PagedAttention" (ghkdgus29.github.io),
sections on basic decoding (filled counts, freeing at the end), parallel sampling
(reference counts, copy-on-write) and scheduling (all-or-nothing eviction, swapping).
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "paged_kv_cache_144_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1", "-fPIC", "-shared"]


def _runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    d = tmp_path_factory.mktemp("sanitize")
    libpa = str(d / "libpa_host_san.so")
    liboracle = str(d / "liboracle_san.so")
    subprocess.run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(CSRC, "block_pool.cpp"), os.path.join(CSRC, "abi.cpp"),
                    os.path.join(HERE, "sanitize_stubs.cpp"), "-o", libpa], check=True)
    subprocess.run(["gcc", "-std=c11", "-fopenmp", *SAN, os.path.join(ROOT, "oracle", "pa_oracle.c"),
                    "-lm", "-o", liboracle], check=True)
    return libpa, liboracle


def test_host_code_clean_under_sanitizers(builds):
    libpa, liboracle = builds
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime()
    # leaks of the interpreter itself are not the library's; every real report aborts
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["OMP_NUM_THREADS"] = "4"
    r = subprocess.run([sys.executable, os.path.join(HERE, "sanitize_run.py"), libpa, liboracle],
                       capture_output=True, text=True, env=env, timeout=1500)
    log = r.stdout + r.stderr
    assert r.returncode == 0, log[-6000:]
    assert "ERROR: AddressSanitizer" not in log and "runtime error:" not in log, log[-6000:]
    assert "[sanitize] clean" in r.stdout
