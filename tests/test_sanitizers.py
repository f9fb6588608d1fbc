"""Sanitizer builds on the CPU (no GPU needed):
  * the host code of libmedusa_hip (tree parsing, sparse-tree search, argument checks, workspace
    sizing) built with AddressSanitizer and UndefinedBehaviorSanitizer on the host side and the
    MEDUSA_CHECKED bounds assertions of its containers, driven by tests/sanitize/
    capi_host_check.cpp over valid, random and malformed inputs;
  * the oracle's C part built with the same sanitizers (gcc), running the oracle pins that call
    it.
A sanitizer report fails the run."""

import concurrent.futures
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "medusa_head_speculative_amd", "csrc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        pytest.skip("hipcc not available")
    return h


def test_capi_host_code_under_asan_ubsan(tmp_path):
    hipcc = _hipcc()
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-DMEDUSA_CHECKED",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), *SAN]
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    srcs.append(os.path.join(ROOT, "tests", "sanitize", "capi_host_check.cpp"))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        p = subprocess.run([hipcc, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert p.returncode == 0, p.stderr
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "capi_host_check")
    p = subprocess.run([hipcc, "--offload-arch=gfx950", *SAN, "-o", exe, *objs],
                       capture_output=True, text=True)
    assert p.returncode == 0, p.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "capi host checks ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_oracle_c_part_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib = str(tmp_path / "liboracle_san.so")
    src = os.path.join(ROOT, "oracle", "medusa_oracle.c")
    subprocess.check_call([gcc, "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-Wall",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", "-o", lib, src, "-lm"])
    asan = subprocess.check_output([gcc, "-print-file-name=libasan.so"], text=True).strip()
    env = dict(os.environ, LD_PRELOAD=asan, MEDUSA_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    tests = [os.path.join(ROOT, "tests", t) for t in
             ("test_oracle_heads.py", "test_oracle_attention.py", "test_oracle_head_blocks.py",
              "test_oracle_rope.py", "test_oracle_commit.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *tests], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
