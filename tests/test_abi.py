"""The C ABI library loads and exports every entry point declared in
include/fftmv.h, and rejects bad arguments before touching a device.
CPU only: no call here reaches a kernel or the HIP runtime."""
import ctypes
import os
import re

import pytest

import fft_block_toeplitz_amd as fm
from fft_block_toeplitz_amd import build as fbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fftmv.h")


@pytest.fixture(scope="module")
def lib():
    if fbuild.is_stale():
        fbuild.build()
    return fm.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fftmv_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(fm.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_only_c_abi_symbols_are_exported(lib):
    out = os.popen(f"nm -D --defined-only {fm.LIB_PATH}").read()
    syms = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert {s for s in syms if s.startswith("fftmv_")} == set(fm.EXPORTS)
    assert not [s for s in syms if "fftmv" in s and not s.startswith("fftmv_")], "internal symbols leak"


def test_status_strings_and_version(lib):
    for st in range(-5, 1):
        assert fm.fftmv_status_string(st)
    assert fm.fftmv_status_string(-99) == "unknown status"
    assert fm.fftmv_version() == (0 << 16) | (1 << 8)


FAKE = 0x10000  # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("args,status", [
    ((0, 8, 4, 16, 0), fm.FFTMV_ERR_INVALID_ARG),               # null F
    ((FAKE + 4, 8, 4, 16, 0), fm.FFTMV_ERR_INVALID_ARG),        # misaligned F
    ((FAKE, 0, 4, 16, 0), fm.FFTMV_ERR_INVALID_ARG),            # Nm < 1
    ((FAKE, 8, 0, 16, 0), fm.FFTMV_ERR_INVALID_ARG),            # Nd < 1
    ((FAKE, 8, 4, 0, 0), fm.FFTMV_ERR_INVALID_ARG),             # Nt < 1
    ((FAKE, 8, 4, 16, 1 << 12), fm.FFTMV_ERR_INVALID_ARG),      # unknown mask bit
    ((FAKE, 8, 4, 2053, 0), fm.FFTMV_ERR_UNSUPPORTED_SIZE),     # prime above 2048: no radix schedule,
                                                                # Bluestein tile too large
    ((FAKE, 8, 4, 2 * 2053, 0), fm.FFTMV_ERR_UNSUPPORTED_SIZE), # the same factor
    ((FAKE, 8, 4, 4093, 0), fm.FFTMV_ERR_UNSUPPORTED_SIZE),     # prime above 2048
    ((FAKE, 8, 4, 5000, 0), fm.FFTMV_ERR_UNSUPPORTED_SIZE),     # Nt > 4096
    ((FAKE, 1 << 31, 4, 16, 0), fm.FFTMV_ERR_UNSUPPORTED_SIZE), # Nm too large
    ((FAKE, (1 << 27) + 1, 4, 16, 0), fm.FFTMV_ERR_UNSUPPORTED_SIZE),  # complex128 row above 2 GiB
])
def test_setup_validates_before_device_work(lib, args, status):
    plan = ctypes.c_void_p(0)
    F, Nm, Nd, Nt, mask = args
    assert lib.fftmv_setup(ctypes.byref(plan), F, Nm, Nd, Nt, mask, None) == status
    assert plan.value is None


def test_null_plan_is_rejected(lib):
    assert lib.fftmv_setup(None, FAKE, 8, 4, 16, 0, None) == fm.FFTMV_ERR_INVALID_ARG
    assert lib.fftmv_apply(None, FAKE, FAKE, None) == fm.FFTMV_ERR_INVALID_ARG
    assert lib.fftmv_apply_adjoint(None, FAKE, FAKE, None) == fm.FFTMV_ERR_INVALID_ARG
    assert lib.fftmv_query(None, None, None) == fm.FFTMV_ERR_INVALID_ARG
    assert lib.fftmv_set_mask(None, 0) == fm.FFTMV_ERR_INVALID_ARG
    assert lib.fftmv_run_stages(None, 0, 1, 5, FAKE, FAKE, None) == fm.FFTMV_ERR_INVALID_ARG
    assert lib.fftmv_buffer(None, 0, None, None, None) == fm.FFTMV_ERR_INVALID_ARG
    assert lib.fftmv_destroy(None) == fm.FFTMV_SUCCESS


def test_mask_constants_follow_stage_numbering():
    assert fm.FFTMV_MIXED_F == fm.FFTMV_FP32(0, 2) | fm.FFTMV_FP32(0, 3)
    assert fm.FFTMV_MIXED_FADJ == fm.FFTMV_FP32(1, 3) | fm.FFTMV_FP32(1, 4)
    assert fm.FFTMV_MIXED == fm.FFTMV_MIXED_F | fm.FFTMV_MIXED_FADJ
    text = open(HEADER).read()
    for name in ("FFTMV_ALL_FP64", "FFTMV_MIXED_F", "FFTMV_MIXED_FADJ", "FFTMV_MIXED", "FFTMV_FLAG_STAGED",
                 "FFTMV_FLAG_FHAT_BOTH", "FFTMV_PREC_BITS"):
        m = re.search(rf"#define {name} \(?(0x[0-9A-Fa-f]+u|1u << \d+)\)?", text)
        assert m, name
        val = eval(m.group(1).replace("u", ""))
        assert val == getattr(fm, name), name
