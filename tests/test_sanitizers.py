"""CPU-only AddressSanitizer + UndefinedBehaviorSanitizer runs.

- The oracle (oracle/oracle.c, built with gcc) under tests/sanitize/
  oracle_driver.c: every entry point on small cases, cross-checked against
  the textbook DFT and the direct sums.
- The host code of libfftmv (every library source built by hipcc with the
  sanitizers on the host side only; device code is unchanged) under
  tests/sanitize/host_driver.cpp: argument validation, plan construction up
  to its first device call, status strings and the precision model. No
  call reaches a kernel; the container has no GPU.

Errors and leaks are fatal (halt_on_error, detect_leaks). Everything is
built in a temporary directory."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from fft_block_toeplitz_amd import build as fbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def run(cmd, env=None, timeout=600):
    res = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout[-4000:]}\n{res.stderr[-4000:]}"
    return res.stdout


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-fopenmp", "-Wall", "-Wextra", os.path.join(ROOT, "oracle", "oracle.c"),
         os.path.join(HERE, "oracle_driver.c"), "-lm", "-o", exe])
    env = dict(os.environ, OMP_NUM_THREADS="4", **SAN_ENV)
    out = run([exe], env=env)
    assert "all checks passed" in out


def test_library_host_code_under_sanitizers(tmp_path):
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(fbuild.HIPCC) and os.path.exists(clangxx)):
        pytest.skip("hipcc / clang++ not available")
    flags = [f"--offload-arch={fbuild.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # sanitizers on the host side only
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             f"-I{os.path.join(ROOT, 'include')}"]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        run([fbuild.HIPCC, *flags, "-c", src, "-o", obj])
        return obj

    workers = max(1, min(len(fbuild.SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(compile_one, fbuild.SOURCES))
    lib = str(tmp_path / "libfftmv_san.so")
    run([fbuild.HIPCC, f"--offload-arch={fbuild.ARCH}", "-shared", "-fPIC",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", *objs, "-o", lib])
    exe = str(tmp_path / "host_san")
    run([clangxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROOT, 'include')}",
         f"-I{os.path.join(ROCM, 'include')}", os.path.join(HERE, "host_driver.cpp"), lib,
         f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64", f"-Wl,-rpath,{tmp_path}",
         f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe])
    out = run([exe], env=dict(os.environ, **SAN_ENV))
    assert "all checks passed" in out
