"""GPU parity at full sizes, in the launch configuration bench.py times.

Main (Nm=5000, Nd=100, Nt=1000; the single-GPU workload of "Mixed-precision
FFTMatvec performance optimization on AMD GPUs", section 4.1): the complete
outputs against the oracle's own five-stage apply (its Fhat built once per
module, 8 GB of complex128 on the host), with the relative L2 error and an
element-wise bound; the complete frequency blocks in both stored
precisions; and, as an independent second check, sampled time steps
against the definition summed directly. The Scale share (Nm=20000, Nd=100,
Nt=2000) is checked on sampled steps from the direct sum. Properties that
hold at any size (adjoint identity, bitwise repeatability) cover the rest.
"""
import sys

import numpy as np
import pytest

import oracle
from fft_block_toeplitz_amd import workloads as W
from parity import within

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def fm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fft_block_toeplitz_amd as fm

    fm.lib()
    return fm


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


class Full:
    def __init__(self, shape, full_oracle=False):
        self.shape = shape
        note(f"generating {shape.name} Nm={shape.Nm} Nd={shape.Nd} Nt={shape.Nt}")
        self.F, self.m, self.d = W.problem(shape)
        self.F_dev = torch.from_numpy(self.F).to("cuda")
        self.m_dev = torch.from_numpy(self.m).to("cuda")
        self.d_dev = torch.from_numpy(self.d).to("cuda")
        Nt = shape.Nt
        self.fsteps = np.array([0, 1, 7, Nt // 2, Nt - 1])
        self.asteps = np.array([0, Nt // 2, Nt - 8, Nt - 2, Nt - 1])
        note("oracle direct sums at spot steps")
        self.v_ref = oracle.direct(self.F, self.m, self.fsteps)
        self.w_ref = oracle.direct_adjoint(self.F, self.d, self.asteps)
        self.Fh = self.v_full = self.w_full = None
        if full_oracle:
            note("oracle setup and five-stage applies (complete outputs)")
            self.Fh = oracle.setup(self.F)
            self.v_full = oracle.apply(self.Fh, self.m)
            self.w_full = oracle.apply_adjoint(self.Fh, self.d)

    def release(self):
        del self.F_dev
        torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def main_case(fm):
    c = Full(W.MAIN, full_oracle=True)
    yield c
    c.release()


def check(fm, c, mask, tol, flags=0, repeat=False):
    plan = fm.Plan(c.F_dev, mask | flags)
    v = host(plan.apply(c.m_dev))
    w = host(plan.apply_adjoint(c.d_dev))
    if c.v_full is not None:
        # the complete outputs against the oracle's five-stage apply
        okv, fv, mv = within(v, c.v_full, tol)
        okw, fw, mw = within(w, c.w_full, tol)
        note(f"{c.shape.name} mask={mask:#05x} flags={flags:#x}: complete outputs rel err F {fv:.3e} F* {fw:.3e}, "
             f"largest entry error / rms F {mv:.2e} F* {mw:.2e}")
        assert okv and okw
    # independent second check: the definition summed directly at spot steps
    okv, ev, mv = within(v[c.fsteps], c.v_ref, tol)
    okw, ew, mw = within(w[c.asteps], c.w_ref, tol)
    ident = abs(np.vdot(v, c.d) - np.vdot(c.m, w)) / (np.linalg.norm(v) * np.linalg.norm(c.d))
    note(f"{c.shape.name} mask={mask:#05x} flags={flags:#x}: spot rel err F {ev:.3e} F* {ew:.3e} "
         f"(entry {mv:.1e}, {mw:.1e}), adjoint identity {ident:.2e}")
    assert okv and okw
    assert ident <= tol
    if repeat:
        assert np.array_equal(v, host(plan.apply(c.m_dev)))
        assert np.array_equal(w, host(plan.apply_adjoint(c.d_dev)))
    plan.close()


def test_main_fhat_complete(fm, main_case):
    """The frequency blocks as the setup builds them at full size, both
    stored precisions, complete, against the oracle's transform."""
    c = main_case
    plan = fm.Plan(c.F_dev, fm.FFTMV_MIXED | fm.FFTMV_FLAG_FHAT_BOTH)
    Nm, Nd, Nt = c.shape.Nm, c.shape.Nd, c.shape.Nt
    for which, tol in ((1, 1e-13), (0, 1e-7)):
        full = plan.read_buffer(which).reshape(Nt + 1, Nd, -1)
        got = full[:, :, :Nm].cpu().numpy()
        pad = full[:, :, Nm:].abs().max().item() if full.shape[2] > Nm else 0.0
        del full
        torch.cuda.empty_cache()
        ok, e, me = within(got, c.Fh, tol)
        del got
        note(f"Fhat {'c128' if which else 'c64'} complete: rel err {e:.3e}, largest entry error / rms {me:.2e}")
        assert ok and pad == 0.0
    plan.close()


def test_main_mixed_as_benchmarked(fm, main_case):
    check(fm, main_case, fm.FFTMV_MIXED, 1e-6, repeat=True)


def test_main_fp64(fm, main_case):
    check(fm, main_case, fm.FFTMV_ALL_FP64, 1e-11)


def test_main_mixed_five_kernel_form(fm, main_case):
    check(fm, main_case, fm.FFTMV_MIXED, 1e-6, flags=fm.FFTMV_FLAG_STAGED)


def test_main_page_masks_separately(fm, main_case):
    """The page's two optimal configurations, each with the other direction
    in FP64 (F̂ held in both precisions)."""
    check(fm, main_case, fm.FFTMV_MIXED_F, 1e-6, flags=fm.FFTMV_FLAG_FHAT_BOTH)
    check(fm, main_case, fm.FFTMV_MIXED_FADJ, 1e-6, flags=fm.FFTMV_FLAG_FHAT_BOTH)


def test_main_fp32_pad_ahead_of_fp64_fft(fm, main_case):
    """Stage 1 in FP32 (input rounded to binary32) ahead of an FP64 FFT, the
    rest FP64: the wide-batch transform with input rounding."""
    mask = fm.FFTMV_FP32(0, 1) | fm.FFTMV_FP32(1, 1)
    check(fm, main_case, mask, 1e-6)


def host_available_bytes():
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemAvailable:"):
                    return int(line.split()[1]) * 1024
    except OSError:
        pass
    return 0


@pytest.mark.slow
def test_scale_share_mixed(fm):
    """One GPU's share of a large grid: Nm=20000, Nd=100, Nt=2000, F̂ ~32 GB
    in complex64. The complete outputs are compared with the oracle's apply
    when the host holds its complex128 F̂ (64 GB) and F (32 GB) twice over;
    the direct-sum spot steps always."""
    if torch.cuda.get_device_properties(0).total_memory < 80 << 30:
        pytest.skip("needs ~70 GB of device memory")
    s = W.SCALE
    need = (s.Nt + 1) * s.Nd * s.Nm * 16 + s.Nt * s.Nd * s.Nm * 8
    full = host_available_bytes() >= 2 * need
    note(f"scale share: complete-output comparison {'on' if full else 'off (host memory)'}")
    c = Full(s, full_oracle=full)
    try:
        check(fm, c, fm.FFTMV_MIXED, 1e-6)
    finally:
        c.release()
