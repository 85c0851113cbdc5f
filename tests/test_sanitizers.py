"""The CPU oracle (oracle/pkv_oracle.c) and the host block allocator
(csrc/block_manager.cpp) rebuilt with gcc's address and undefined-behaviour
sanitizers, and the existing oracle and allocator batteries run against those
builds in a child process (the ASan runtime is preloaded there, since the Python
interpreter itself is not instrumented).  Any out-of-bounds access, use after
free, double free, signed overflow or misaligned access the batteries reach
aborts the child and fails this test.  CPU only."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

BATTERIES = ["tests/sanitize/test_sanitized_builds_loaded.py", "tests/test_oracle.py", "tests/test_oracle_mutants.py", "tests/test_block_manager.py",
             "tests/test_block_manager_oracle.py", "tests/test_index_checks.py"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


@pytest.fixture(scope="module")
def sanitized_libs(tmp_path_factory):
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("another library is preloaded; the ASan runtime must come first")
    for tool in ("gcc", "g++"):
        if shutil.which(tool) is None:
            pytest.skip(f"{tool} not found")
    out = tmp_path_factory.mktemp("san")
    orc = str(out / "liboracle_asan.so")
    _run(["gcc", *SAN, "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", orc,
          os.path.join(ROOT, "oracle", "pkv_oracle.c"), "-lm"])
    blk = str(out / "libblocks_asan.so")
    csrc = os.path.join(ROOT, "paged_kv_cache_80_amd", "csrc")
    _run(["g++", *SAN, "-std=c++17", "-fPIC", "-shared", f"-I{os.path.join(ROOT, 'include')}", f"-I{csrc}",
          "-o", blk, os.path.join(csrc, "block_manager.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "last_error_stub.cpp")])
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc has no shared ASan runtime")
    return orc, blk, asan


def test_batteries_under_asan_and_ubsan(sanitized_libs):
    orc, blk, asan = sanitized_libs
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, PKV_TEST_ORACLE_LIB=orc, PKV_TEST_BLOCKS_LIB=blk, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu", *BATTERIES]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail


def test_sanitizers_catch_a_planted_overflow(sanitized_libs, tmp_path):
    """The same flags catch a one-element heap overflow: the net is live, not silent."""
    src = tmp_path / "bad.c"
    src.write_text("#include <stdlib.h>\nint main(void){int*a=malloc(4*sizeof(int));a[4]=1;int r=a[4];"
                   "free(a);return r;}\n")
    exe = str(tmp_path / "bad")
    _run(["gcc", *SAN, "-o", exe, str(src)])
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode != 0 and ("heap-buffer-overflow" in r.stderr or "runtime error" in r.stderr)
