"""Build libfftmv.so (HIP, gfx950) in-tree with hipcc."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfftmv.so")
SOURCES = [os.path.join(HERE, "csrc", f)
           for f in ("fft_generic_fwd.hip", "fft_generic_inv.hip", "fft_generic_fwd_blue.hip",
                     "fft_generic_inv_blue.hip", "fft_fixed_fwd.hip", "fft_fixed_inv.hip", "fft_setup.hip", "sbgemv.hip",
                     "padcast.hip", "condition.hip", "scratch.hip", "plan.cpp", "precision.cpp")]
# measurement kernels of the benchmark (memory ceilings): a library of their own
CEILING_SRC = os.path.join(HERE, "csrc", "ceiling.hip")
CEILING_LIB = os.path.join(HERE, "libfftmv_ceiling.so")
HEADERS = [os.path.join(ROOT, "include", "fftmv.h")] + [
    os.path.join(HERE, "csrc", f) for f in ("common.hpp", "internal.hpp", "fft_device.hpp", "fft_fixed.hpp",
                                            "fft_generic.hpp")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
    # no packed FP32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False) -> str:
    """Compile every HIP source (in parallel) and link
    fft_block_toeplitz_amd/libfftmv.so, and the benchmark's memory-ceiling
    kernels into fft_block_toeplitz_amd/libfftmv_ceiling.so."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    noise = "packed-fp32-ops"  # the host pass does not know this device feature
    inc = f"-I{os.path.join(ROOT, 'include')}"
    with tempfile.TemporaryDirectory(prefix="fftmv_build_") as tmpdir:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [HIPCC, *FLAGS, inc, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            return obj, subprocess.run(cmd, capture_output=True, text=True)

        workers = max(1, min(len(SOURCES) + 1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(workers) as ex:
            results = list(ex.map(compile_one, SOURCES + [CEILING_SRC]))
        ceiling_obj, ceiling_res = results.pop()
        results_all = results + [(ceiling_obj, ceiling_res)]
        msgs = []
        for (obj, res), src in zip(results_all, SOURCES + [CEILING_SRC]):
            out = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and ln.strip()]
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(out))
            msgs += out
        tmp = LIB + f".tmp{os.getpid()}"
        cmd = [HIPCC, *FLAGS, "-shared", *[o for o, _ in results], "-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
        ctmp = CEILING_LIB + f".tmp{os.getpid()}"
        res = subprocess.run([HIPCC, *FLAGS, "-shared", ceiling_obj, "-o", ctmp], capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed (ceiling kernels):\n" + res.stdout + res.stderr)
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    os.replace(ctmp, CEILING_LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB) or not os.path.exists(CEILING_LIB):
        return True
    t = min(os.path.getmtime(LIB), os.path.getmtime(CEILING_LIB))
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS + [CEILING_SRC])


if __name__ == "__main__":
    print(build(verbose=True))
