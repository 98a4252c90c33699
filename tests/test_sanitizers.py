"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer: the fp64
oracle (every pin) and the host KV block allocator (a seeded call sequence
against its model, error paths and the serving run).  Each is compiled by g++
with the sanitizers into a temporary library and exercised in a child process
that preloads the ASan runtime; any report fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-std=c++17", "-fPIC", "-shared", "-pthread"]


def asan_runtime():
    p = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if p and os.path.isabs(p) and os.path.exists(p) else None


def run_sanitized(kind, lib):
    env = dict(os.environ, LD_PRELOAD=asan_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitized_run.py"), kind, lib], env=env,
                       capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


@pytest.fixture(scope="module")
def runtime():
    if asan_runtime() is None:
        pytest.skip("g++ has no ASan runtime")


def test_oracle_under_sanitizers(runtime, tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["g++", *SAN, os.path.join(ROOT, "oracle", "oracle.cpp"), "-o", lib], check=True)
    out = run_sanitized("oracle", lib)
    assert out.count("pin ok:") >= 20


def test_allocator_under_sanitizers(runtime, tmp_path):
    lib = str(tmp_path / "liballoc_san.so")
    subprocess.run(["g++", *SAN, "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    "-D__HIP_PLATFORM_AMD__", os.path.join(ROOT, "paged_kv_gqa_slot_amd", "csrc", "kv_allocator.cpp"),
                    "-o", lib], check=True)
    out = run_sanitized("allocator", lib)
    assert "allocator ok" in out
